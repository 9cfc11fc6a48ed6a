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
    if kernel not in KERNEL_SOURCES:
        return None
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
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other workloads (single linear, decoder step, layer slices)")
    p.add_argument("--config-steps", type=int, default=20)
    p.add_argument("--only-config", default="",
                   help="with --kernel-only configs: only the workloads whose name starts so "
                        "(e.g. decoder32_7b_b1_s40, slice_13b)")
    p.add_argument("--kernel-only", choices=["", "gather", "topk1", "topk1s", "topk2", "fused1",
                                             "step", "copy", "configs"],
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
    if a.kernel_only == "configs":
        print(json.dumps(other_configs(a, dev)), flush=True)
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
    ws_mlp = torch.zeros(_lib.larosa_mlp_workspace_bytes(1, d, f, case.k1, case.k2, _lib.FUSED),
                         dtype=torch.uint8, device=dev)

    def step(i, mode):
        # one call for the whole MLP: in unfused mode 4 launches (rotate x;
        # the gate|up product with the selection and SiLU(gate)·up folded in;
        # rotate h; the down product), in fused mode 2 one-launch layers
        c = i % copies
        _lib.larosa_mlp_forward(x_d, qt1[c], l1.q_block, wil1[c], qt2[c], l2.q_block, wf2[c], 1,
                                d, f, case.k1, case.k2, h, y, mode=mode, ws=ws_mlp)

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
    # the chained form (the rotation of h inside the gate|up launch), eager
    chain_ms = timed(lambda i: step(i, _lib.CHAIN), a.steps, a.warmup) \
        if a.kernel_only == "" else None

    def per_step_us(fn, steps):
        # an event pair around every step (the steps still run back to back):
        # the spread of single-step device times
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i, (s0, s1) in enumerate(evs):
            s0.record(stream)
            fn(i)
            s1.record(stream)
        torch.cuda.synchronize()
        t = sorted(s0.elapsed_time(s1) * 1e3 for s0, s1 in evs)

        def pct(p):
            return round(t[min(len(t) - 1, int(round(p / 100 * (len(t) - 1))))], 2)
        return {"median": pct(50), "p10": pct(10), "p90": pct(90), "steps": steps}

    step_dist = {name: per_step_us(lambda i, m=modes[name]: step(i, m), max(a.steps, 100))
                 for name in eager_ms} if a.kernel_only == "" else {}

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

    def topk1s(i):  # the gate|up kernel with SiLU(gate)·up folded in
        _lib.larosa_topk_swiglu_gemv(xr1, d, case.k1, wil1[i % copies], h, f, ws=ws1)

    def chain1(i):  # the chained form's gate|up kernel: SwiGLU product, then Q2's rotation
        c = i % copies
        _lib.larosa_topk_swiglu_rotate(xr1, d, case.k1, wil1[c], h, f, qt2[c], l2.q_block, xr2,
                                       ws=ws1)

    def topk2(i):
        _lib.larosa_topk_gemv(xr2, f, case.k2, wf2[i % copies], y, d, ws=ws2)

    def gather(i):
        _lib.larosa_sparse_gemv(idx1, None, case.k1, val1, wf1[i % copies], gu, 1, d, 2 * f,
                                ws=ws1)

    def fused1(i):
        c = i % copies
        _lib.larosa_layer_forward(x_d, qt1[c], l1.q_block, wf1[c], 1, d, 2 * f, case.k1, gu,
                                  mode=_lib.FUSED, ws=ws1)
    if a.kernel_only in ("gather", "topk1", "topk1s", "chain1", "topk2", "fused1"):
        fn = {"gather": gather, "topk1": topk1, "topk1s": topk1s, "chain1": chain1,
              "topk2": topk2, "fused1": fused1}[a.kernel_only]
        for i in range(a.steps):
            fn(i)
        torch.cuda.synchronize()
        return
    topk1_ms = timed(topk1, a.steps, a.warmup)
    topk1_bytes = case.k1 * 2 * f * 2 + d * 4 + 2 * f * 2
    topk1s_ms = timed(topk1s, a.steps, a.warmup)
    topk1s_bytes = case.k1 * 2 * f * 2 + d * 4 + f * 2
    topk2_ms = timed(topk2, a.steps, a.warmup)
    topk2_bytes = case.k2 * d * 2 + f * 4 + d * 2
    chain1_ms = timed(chain1, a.steps, a.warmup)
    # kept gate|up rows, x_rot, h written and read back, Q2, x_rot2
    chain1_bytes = case.k1 * 2 * f * 2 + d * 4 + 2 * f * 2 + l2.Qt.numel() * 2 + f * 4
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

    def gbs(nbytes, ms_):
        return nbytes / (ms_ * 1e-3) / 1e9

    # The dense MLP step on the same GPU: dense gate|up, SiLU(gate)·up, dense
    # down, over weights of the same shapes (cycling the same copies), with
    # the faster of this library's dense product and torch.matmul.
    ws_d2 = torch.zeros(_lib.larosa_workspace_bytes(1, f, d, f, _lib.UNFUSED), dtype=torch.uint8,
                        device=dev)

    def dense_mlp(i, use_torch):
        c = i % copies
        if use_torch:
            torch.matmul(x_d, wf1[c], out=gu)
            _lib.larosa_swiglu(gu, h, 1, f)
            torch.matmul(h, wf2[c], out=y)
        else:
            _lib.larosa_dense_gemv(x_d, wf1[c], gu, 1, d, 2 * f, ws=ws1)
            _lib.larosa_swiglu(gu, h, 1, f)
            _lib.larosa_dense_gemv(h, wf2[c], y, 1, f, d, ws=ws_d2)
    dense_mlp_ms = {
        "larosa_dense_gemv": timed(lambda i: dense_mlp(i, False), a.steps, a.warmup),
        "torch.matmul": timed(lambda i: dense_mlp(i, True), a.steps, a.warmup),
    }
    copy = copy_ceiling(dev, timed, a.steps, a.warmup)

    # Per-stage times of the unfused step (each stage alone, cycling copies).
    stage = {}
    stage["rotate1"] = timed(lambda i: _lib.larosa_rotate(x_d, qt1[i % copies], l1.q_block, xr1,
                                                          1, d), a.steps, a.warmup)
    stage["select_gather1"] = topk1s_ms
    stage["swiglu_alone"] = timed(lambda i: _lib.larosa_swiglu(gu, h, 1, f), a.steps, a.warmup)
    stage["rotate2"] = timed(lambda i: _lib.larosa_rotate(h, qt2[i % copies], l2.q_block, xr2,
                                                          1, f), a.steps, a.warmup)
    stage["select_gather2"] = timed(topk2, a.steps, a.warmup)
    stage["select1_alone"] = timed(lambda i: _lib.larosa_topk_select(xr1, 1, d, case.k1, idx1,
                                                                     val1), a.steps, a.warmup)
    stage["gather1_alone"] = gather_ms

    # The fp64-accumulating rotation beside the fp32 one, for both rotations
    # of the MLP at 1, 4 and 8 tokens, and the one-token step with it.
    exact_rot = {}
    for nb in (1, 4, 8):
        for tag, src, lin, dd, dst_d in (("q1", x_d, l1, d, xr1), ("q2", h, l2, f, xr2)):
            xb = src.expand(nb, dd).contiguous()
            dst = dst_d if nb == 1 else torch.empty((nb, dd), dtype=torch.float32, device=dev)
            qts = qt1 if tag == "q1" else qt2
            for prec, fn in (("fp32", _lib.larosa_rotate), ("fp64", _lib.larosa_rotate_fp64)):
                t = timed(lambda i, fn=fn, xb=xb, dst=dst, qts=qts, lin=lin, nb=nb, dd=dd:
                          fn(xb, qts[i % copies], lin.q_block, dst, nb, dd), a.steps, a.warmup)
                nbytes = lin.Qt.numel() * 2 + nb * dd * (2 + 4)
                exact_rot[f"{tag}_b{nb}_{prec}"] = {"us": round(t * 1e3, 2),
                                                    "GBs": round(gbs(nbytes, t), 1)}
    exact_rot["step_ms_unfused_fp64_rotation"] = round(
        timed(lambda i: step(i, _lib.UNFUSED | _lib.ROTATE_FP64), a.steps, a.warmup), 5)

    thr = threshold_mlp(a, case, x_d, l1, l2, qt1, wil1, qt2, wf2, copies, h, y, timed, gbs)
    lowr = lowrank_gate_up(a, case, x_d, l1, qt1, wf1, copies, timed, gbs)
    sweep = q2_block_sweep(a, case, wd, l1, x_d, qt1, wil1, copies, h, y, timed, gbs)

    q_bytes = (l1.Qt.numel() + l2.Qt.numel()) * 2
    sparse_bytes = q_bytes + (case.k1 * 2 * f + case.k2 * d) * 2
    dense_mlp_bytes = (d * 2 * f + f * d) * 2
    best = min(step_ms, key=step_ms.get)
    ms = step_ms[best]
    rot1_bytes = l1.Qt.numel() * 2 + d * 2 + d * 4
    rot2_bytes = l2.Qt.numel() * 2 + f * 2 + f * 4
    kernels = {
        "select_gather_kernel": dict(
            achieved=gbs(topk1s_bytes, topk1s_ms), bytes=topk1s_bytes, us=topk1s_ms * 1e3,
            what="one-token selection folded into the gate|up product with SiLU(gate)·up "
                 "(the step's largest kernel)"),
        "select_gather_kernel (chained)": dict(
            achieved=gbs(chain1_bytes, chain1_ms), bytes=chain1_bytes, us=chain1_ms * 1e3,
            what="the same product chained into the rotation of h by Q2 (LAROSA_CHAIN)"),
        "select_gather_kernel (no epilogue)": dict(
            achieved=gbs(topk1_bytes, topk1_ms), bytes=topk1_bytes, us=topk1_ms * 1e3,
            what="the same selection and product writing gate|up"),
        "select_gather_kernel (down)": dict(
            achieved=gbs(topk2_bytes, topk2_ms), bytes=topk2_bytes, us=topk2_ms * 1e3,
            what="one-token selection folded into the product, down (11008 -> 4096)"),
        "rotate_row_kernel (Q1)": dict(
            achieved=gbs(rot1_bytes, stage["rotate1"]), bytes=rot1_bytes,
            us=stage["rotate1"] * 1e3, what="one-token rotation, dense 4096x4096"),
        "rotate_row_kernel (Q2)": dict(
            achieved=gbs(rot2_bytes, stage["rotate2"]), bytes=rot2_bytes,
            us=stage["rotate2"] * 1e3, what=f"one-token rotation, {f // case.q2_block}x"
                                            f"{case.q2_block} blocks"),
        "gather_vec_kernel": dict(achieved=gbs(gather_bytes, gather_ms), bytes=gather_bytes,
                                  us=gather_ms * 1e3,
                                  what="product over a given kept-row list, gate|up"),
        "fused_linear_kernel": dict(achieved=gbs(fused1_bytes, fused1_ms), bytes=fused1_bytes,
                                    us=fused1_ms * 1e3, what="fused rotate-select-gather, gate|up"),
    }
    dom = "fused_linear_kernel" if best == "fused" else "select_gather_kernel"
    kd = kernels[dom]

    configs = None
    if not a.no_configs:
        # the MLP's copies are no longer needed
        del qt1, wf1, wil1, qt2, wf2
        torch.cuda.empty_cache()
        configs = other_configs(a, dev)

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
            "step": "larosa_mlp_forward (unfused: 4 launches, rotate x, gate|up product with "
                    "the selection and SiLU(gate)·up folded in, rotate h, down product; fused: "
                    "the two one-launch layer calls)",
            "chain_step_ms_eager": round(chain_ms, 5) if chain_ms else None,
            "eager_step_ms": {k: round(v, 5) for k, v in eager_ms.items()},
            "graph_step_ms": {k: round(v, 5) for k, v in graph_ms.items()},
            "eager_step_us_per_step_events": step_dist,
            "mlp_sparse_bytes": sparse_bytes,
            "mlp_dense_weight_bytes": dense_mlp_bytes,
            "mlp_achieved_GBs": round(sparse_bytes / (ms * 1e-3) / 1e9, 1),
            "stage_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
            "rotation_fp32_vs_fp64": exact_rot,
            "threshold_select": thr,
            "lowrank_compensation": lowr,
            "q2_block_sweep": sweep,
            "kernels": {k: {"achieved_GBs": round(v["achieved"], 1), "bytes_per_launch": v["bytes"],
                            "avg_us": round(v["us"], 3), "frac": round(v["achieved"] / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(k)} for k, v in kernels.items()},
            "gate_up_dense_us": {"larosa_dense_gemv": round(dense_ms * 1e3, 2),
                                 "torch.matmul": round(torch_ms * 1e3, 2)},
            "gate_up_dense_GBs": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1),
            "gate_up_speedup_vs_dense": round(min(dense_ms, torch_ms) / topk1_ms, 3),
            "down_select_gather_frac_of_peak": round(gbs(topk2_bytes, topk2_ms) / HBM_PEAK_GBS, 4),
            "gate_up_speedup_note": "the product alone (selection folded in), without the "
                                    "rotation; the MLP-level figure is step_speedup_vs_dense",
            "mlp_dense_step_ms": {k: round(v, 5) for k, v in dense_mlp_ms.items()},
            "step_speedup_vs_dense": round(min(dense_mlp_ms.values()) / ms, 3),
            "step_speedup_vs_dense_q2_256": (
                round(min(dense_mlp_ms.values()) / sweep["256"]["step_ms"], 3)
                if "256" in sweep else None),
            "copy_ceiling": copy,
            "roofline_frac_of_copy_ceiling": round(kd["achieved"] / copy["GBs"], 4),
            "gate_up_gather_only_speedup_vs_dense": round(min(dense_ms, torch_ms) / gather_ms, 3),
            "input_gen_s": round(gen_s, 1),
            "configs": configs,
        },
    }
    print(json.dumps(out), flush=True)


def threshold_mlp(a, case, x_d, l1, l2, qt1, wil1, qt2, wf2, copies, h, y, timed, gbs):
    """The same one-token MLP with the magnitude-threshold selection in place
    of the Top-K: t1 and t2 are calibrated on the device from 64 synthetic
    calibration tokens (t2 on the h those tokens produce), then one decode
    step is timed, and the kept counts of 64 further tokens are reported
    (the per-token sparsity that a threshold lets fluctuate)."""
    import torch
    from rotated_top_activation_amd import _lib, workloads as wl
    dev = x_d.device
    d, f, p = case.d, case.f, a.sparsity
    n_cal = 64
    cal_ws = torch.empty(_lib.larosa_calibrate_workspace_bytes(), dtype=torch.uint8, device=dev)
    t_d = torch.empty(2, dtype=torch.float32, device=dev)

    def batch_ws(B, d_in, f_):
        return torch.zeros(_lib.larosa_swiglu_workspace_bytes(B, d_in, f_, d_in, _lib.UNFUSED),
                           dtype=torch.uint8, device=dev)

    def down_ws(B):
        return torch.zeros(_lib.larosa_workspace_bytes(B, f, d, f, _lib.UNFUSED),
                           dtype=torch.uint8, device=dev)

    def run_batch(xb, t1, t2):
        B = xb.shape[0]
        hb = torch.empty((B, f), dtype=torch.bfloat16, device=dev)
        yb = torch.empty((B, d), dtype=torch.bfloat16, device=dev)
        c1 = torch.empty(B, dtype=torch.int32, device=dev)
        c2 = torch.empty(B, dtype=torch.int32, device=dev)
        _lib.larosa_threshold_swiglu_layer_forward(xb, l1.Qt, l1.q_block, wil1[0], B, d, f, t1,
                                                   hb, count_out=c1, ws=batch_ws(B, d, f))
        if t2 is not None:
            _lib.larosa_threshold_layer_forward(hb, l2.Qt, l2.q_block, wf2[0], B, f, d, t2, yb,
                                                count_out=c2, ws=down_ws(B))
        return hb, c1, c2

    # calibration
    x_cal = wl.to_torch(wl.heavy_tailed_activations(2, 0, "mlp_in", n_cal, d, "bf16",
                                                    run_seed=17), "bf16")
    xr_cal = torch.empty((n_cal, d), dtype=torch.float32, device=dev)
    _lib.larosa_rotate(x_cal, l1.Qt, l1.q_block, xr_cal, n_cal, d)
    _lib.larosa_calibrate_threshold(xr_cal, n_cal * d, n_cal * d * (100 - p) // 100, t_d[0:1],
                                    cal_ws)
    t1 = float(t_d[0].item())
    h_cal, _, _ = run_batch(x_cal, t1, None)
    hr_cal = torch.empty((n_cal, f), dtype=torch.float32, device=dev)
    _lib.larosa_rotate(h_cal, l2.Qt, l2.q_block, hr_cal, n_cal, f)
    _lib.larosa_calibrate_threshold(hr_cal, n_cal * f, n_cal * f * (100 - p) // 100, t_d[1:2],
                                    cal_ws)
    t2 = float(t_d[1].item())

    # one decode step
    ws1 = batch_ws(1, d, f)
    ws2 = down_ws(1)
    cnt = torch.empty(2, dtype=torch.int32, device=dev)

    def step(i, counts=False):
        c = i % copies
        _lib.larosa_threshold_swiglu_layer_forward(x_d, qt1[c], l1.q_block, wil1[c], 1, d, f, t1,
                                                   h, count_out=cnt[0:1] if counts else None,
                                                   ws=ws1)
        _lib.larosa_threshold_layer_forward(h, qt2[c], l2.q_block, wf2[c], 1, f, d, t2, y,
                                            count_out=cnt[1:2] if counts else None, ws=ws2)
    step(0, counts=True)
    torch.cuda.synchronize()
    k1, k2 = (int(v) for v in cnt.tolist())
    step_ms = timed(step, a.steps, a.warmup)
    xr1 = torch.empty((1, d), dtype=torch.float32, device=dev)
    _lib.larosa_rotate(x_d, l1.Qt, l1.q_block, xr1, 1, d)
    gu = torch.empty((1, 2 * f), dtype=torch.bfloat16, device=dev)
    ws_g = torch.zeros(_lib.larosa_workspace_bytes(1, d, 2 * f, d, _lib.UNFUSED),
                       dtype=torch.uint8, device=dev)
    # the folded selection + product alone (gate|up, without SwiGLU): the
    # threshold form of the Top-K kernel timed in stage_us["select_gather1"]
    sg_ms = timed(lambda i: _lib.larosa_threshold_layer_forward(
        x_d, qt1[i % copies], l1.q_block, wil1[i % copies], 1, d, 2 * f, t1, gu, ws=ws_g),
        a.steps, a.warmup)
    rot_ms = timed(lambda i: _lib.larosa_rotate(x_d, qt1[i % copies], l1.q_block, xr1, 1, d),
                   a.steps, a.warmup)
    sg_only_ms = max(sg_ms - rot_ms, 1e-6)
    sg_bytes = k1 * 2 * f * 2 + d * 4 + 2 * f * 2

    # kept counts of 64 more tokens
    x_test = wl.to_torch(wl.heavy_tailed_activations(2, 0, "mlp_in", 64, d, "bf16",
                                                     run_seed=18), "bf16")
    _, c1, c2 = run_batch(x_test, t1, t2)
    c1 = c1.cpu().numpy()
    c2 = c2.cpu().numpy()
    q_bytes = (l1.Qt.numel() + l2.Qt.numel()) * 2
    step_bytes = q_bytes + (k1 * 2 * f + k2 * d) * 2
    return {
        "calibration": f"t = the floor(n*(100-p)/100)-th largest |x_rot| over {n_cal} synthetic "
                       f"tokens (n = {n_cal}*d), on the device; t2 on those tokens' h",
        "t1": t1, "t2": t2,
        "step_ms": round(step_ms, 5),
        "step_tokens_per_s": round(1.0 / (step_ms * 1e-3), 2),
        "step_kept": {"gate_up_in": k1, "down_in": k2},
        "step_GBs": round(gbs(step_bytes, step_ms), 1),
        "gate_up_select_gather_us_layer_minus_rotation": round(sg_only_ms * 1e3, 2),
        "gate_up_select_gather_GBs": round(gbs(sg_bytes, sg_only_ms), 1),
        "kept_64_tokens": {
            "gate_up_in": {"min": int(c1.min()), "mean": round(float(c1.mean()), 1),
                           "max": int(c1.max()), "top_k": case.k1},
            "down_in": {"min": int(c2.min()), "mean": round(float(c2.mean()), 1),
                        "max": int(c2.max()), "top_k": case.k2},
        },
    }


def copy_ceiling(dev, timed, steps, warmup, nbytes=1 << 30):
    """A plain device-to-device copy of nbytes (read once, written once):
    the practical HBM ceiling on this part, next to the 8 TB/s peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    ms = timed(lambda i: dst.copy_(src), max(20, steps // 4), max(3, warmup // 4))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read_plus_written": 2 * nbytes, "us": round(ms * 1e3, 2),
            "GBs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def q2_block_sweep(a, case, wd, l1, x_d, qt1, wil1, copies, h, y, timed, gbs,
                   blocks=(256, 688, 1376, 2752, 5504, 11008), steps=100, repeats=3):
    """The one-token MLP step with the down projection's rotation Q2 made of
    f / b independent b×b Haar blocks, for block widths b that divide f =
    11008 (the pages allow any orthogonal rotation, random or learned): the
    Q2 bytes fall as b shrinks. Q2 drawn on the device (QR of a seeded N(0,1)
    matrix, sign-fixed), folded into the same W_down; three copies per point
    so the on-package cache serves none of a step's reads. Each point is the
    median of `repeats` timings of at least `steps` steps, whatever the
    command line's step count."""
    import torch
    from rotated_top_activation_amd import _lib
    from rotated_top_activation_amd.device import RotatedLinear
    dev = x_d.device
    d, f = case.d, case.f
    gen = torch.Generator(device=dev)
    ws_mlp = torch.zeros(_lib.larosa_mlp_workspace_bytes(1, d, f, case.k1, case.k2,
                                                         _lib.UNFUSED),
                         dtype=torch.uint8, device=dev)
    w_down = None
    out = {}
    for b in blocks:
        if f % b:
            continue
        gen.manual_seed(1000 + b)
        lins = []
        for _ in range(3):
            q = _dev_haar(gen, b, f // b, dev)
            if w_down is None:
                w_down = wl_to_dev(wd)
            lins.append(RotatedLinear(q, w_down, "bf16", case.k2, keep_w=False))
        xr2 = torch.empty((1, f), dtype=torch.float32, device=dev)

        def step(i, lins=lins, b=b):
            c = i % copies
            l2 = lins[i % 3]
            _lib.larosa_mlp_forward(x_d, qt1[c], l1.q_block, wil1[c], l2.Qt, b, l2.Wf, 1, d, f,
                                    case.k1, case.k2, h, y, ws=ws_mlp)
        n_steps = max(steps, a.steps)
        runs = sorted(timed(step, n_steps, max(a.warmup, 10)) for _ in range(repeats))
        ms = runs[len(runs) // 2]
        rot = sorted(timed(lambda i, lins=lins, b=b: _lib.larosa_rotate(h, lins[i % 3].Qt, b, xr2,
                                                                        1, f),
                           n_steps, max(a.warmup, 10)) for _ in range(repeats))[repeats // 2]
        q_bytes = l1.Qt.numel() * 2 + f * b * 2
        sparse = q_bytes + (case.k1 * 2 * f + case.k2 * d) * 2
        dense = (d * 2 * f + f * d) * 2
        out[str(b)] = {"step_ms": round(ms, 5), "step_ms_runs": [round(r, 5) for r in runs],
                       "steps_per_run": n_steps,
                       "tokens_per_s": round(1.0 / (ms * 1e-3), 1),
                       "rotate2_us": round(rot * 1e3, 2), "q2_bytes": f * b * 2,
                       "step_bytes": sparse, "step_GBs": round(gbs(sparse, ms), 1),
                       "dense_over_sparse_bytes": round(dense / sparse, 3)}
        del lins
        torch.cuda.empty_cache()
    return out


def wl_to_dev(w):
    from rotated_top_activation_amd import workloads as wl
    return wl.to_torch(w, "bf16")


def lowrank_gate_up(a, case, x_d, l1, qt1, wf1, copies, timed, gbs, r=64):
    """The gate|up linear with rank-r compensation of the dropped channels:
    y = xs·W' + (x_rot − xs)·A_r·B_r, factors from a randomised SVD of the
    folded weight on the device (offline, untimed), B_r stored below each
    weight copy. Timed beside the plain Top-K layer on the same copies."""
    import torch
    from rotated_top_activation_amd import _lib
    dev = x_d.device
    d, n = case.d, 2 * case.f
    torch.manual_seed(0)
    u, sv, v = torch.svd_lowrank(l1.Wf.float(), q=r + 16, niter=3)
    root = sv[:r].sqrt()
    a_r = (u[:, :r] * root[None, :]).to(torch.bfloat16).contiguous()
    b_r = (root[:, None] * v[:, :r].T).to(torch.bfloat16).contiguous()
    w_ext = [torch.cat([wf1[c], b_r], dim=0).contiguous() for c in range(copies)]
    gu = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(_lib.larosa_lowrank_workspace_bytes(1, d, n, case.k1, r), dtype=torch.uint8,
                     device=dev)
    ws_plain = torch.zeros(_lib.larosa_workspace_bytes(1, d, n, case.k1, _lib.UNFUSED),
                           dtype=torch.uint8, device=dev)
    lr_ms = timed(lambda i: _lib.larosa_lowrank_layer_forward(
        x_d, qt1[i % copies], l1.q_block, w_ext[i % copies], a_r, r, 1, d, n, case.k1, gu, ws=ws),
        a.steps, a.warmup)
    plain_ms = timed(lambda i: _lib.larosa_layer_forward(
        x_d, qt1[i % copies], l1.q_block, wf1[i % copies], 1, d, n, case.k1, gu, ws=ws_plain),
        a.steps, a.warmup)
    nbytes = l1.Qt.numel() * 2 + (case.k1 + r) * n * 2 + d * r * 2
    del w_ext
    return {
        "rank": r, "factors": "randomised SVD of W'_gate|up on the device (offline)",
        "gate_up_layer_us": round(lr_ms * 1e3, 2),
        "gate_up_layer_GBs": round(gbs(nbytes, lr_ms), 1),
        "plain_top_k_layer_us": round(plain_ms * 1e3, 2),
        "extra_bytes": (r * n + d * r) * 2,
    }


# ---------------------------------------------------------------- other workloads --
# The single fp32 linear, the 32-layer decoder step and the 13B / 70B layer
# slices, timed with HIP events like the MLP. Their rotations and weights are
# drawn on the device (QR of a seeded N(0,1) matrix, sign-fixed; seeded
# Gaussian weights): the same distributions as the test inputs, without the
# host QR of 8192² matrices. Bytes per step are what the path must read: the
# rotations, the union rows of every folded weight (union sizes from one
# traced step) and, for the decoder, the key/value cache.

def _dev_haar(gen, n: int, nb: int, device):
    import torch
    out = []
    for _ in range(nb):
        g = torch.randn((n, n), generator=gen, device=device, dtype=torch.float32)
        q, r = torch.linalg.qr(g)
        sg = torch.sign(torch.diagonal(r))
        sg[sg == 0] = 1.0
        out.append((q * sg[None, :]).to(torch.bfloat16))
    return torch.stack(out)


def _dev_weight(gen, d_in: int, d_out: int, std: float, device):
    import torch
    return (torch.randn((d_in, d_out), generator=gen, device=device) * std).to(torch.bfloat16)


def _timed_ms(fn, steps: int, warmup: int) -> float:
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _union_rows(idx) -> int:
    import torch
    return int(torch.unique(idx.reshape(-1)).numel())


def _entry(B, ms, nbytes, extra=None):
    out = {"tokens_per_s": round(B / (ms * 1e-3), 1), "us_per_step": round(ms * 1e3, 2),
           "bytes_per_step": int(nbytes), "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if extra:
        out.update(extra)
    return out


def _single_linear_f32(res, device):
    """The fp32 512 -> 1536 single linear at batch 1, 40%, both modes."""
    import torch
    from rotated_top_activation_amd import _lib, workloads as wl
    from rotated_top_activation_amd.device import RotatedLinear
    case, x, q, w = wl.single_linear_f32()
    lin = RotatedLinear(q, w, "f32", case.k)
    x_d = wl.to_torch(x, "f32")
    y = torch.empty((1, 1536), dtype=torch.float32, device=device)
    best = None
    for mode, name in ((_lib.UNFUSED, "unfused"), (_lib.FUSED, "fused")):
        ws = lin.workspace(1, mode)
        ms = _timed_ms(lambda: lin.forward(x_d, y, ws, mode=mode), 200, 20)
        if best is None or ms < best[0]:
            best = (ms, name)
    nbytes = 512 * 512 * 4 + case.k * 1536 * 4
    res["single_linear_f32_512x1536_b1_s40"] = _entry(1, best[0], nbytes, {"mode": best[1]})
    del lin


def other_configs(a, device):
    import torch
    from rotated_top_activation_amd import _lib, decoder as dec, workloads as wl
    from rotated_top_activation_amd.device import RotatedLinear
    steps, warm = a.config_steps, 3
    res = {}
    only = getattr(a, "only_config", "")

    def want(name):
        return not only or name.startswith(only)

    # single linear, fp32, 512 -> 1536, batch 1, 40%
    if want("single_linear_f32_512x1536_b1_s40"):
        _single_linear_f32(res, device)

    # 32-layer 7B decoder step
    if any(want(f"decoder32_7b_b{B}_s{sp}") for B in (1, 4, 16) for sp in (25, 40, 50)):
        shape = wl.LLAMA7B
        gen = torch.Generator(device=device)
        gen.manual_seed(3)
        d, f = shape.d, shape.f
        base = {
            "q_attn": _dev_haar(gen, d, 1, device), "q_o": _dev_haar(gen, d, 1, device),
            "q_mlp": _dev_haar(gen, d, 1, device),
            "q_down": _dev_haar(gen, shape.q2_block, f // shape.q2_block, device),
            "w_qkv": _dev_weight(gen, d, shape.qkv_out, shape.w_std, device),
            "w_o": _dev_weight(gen, d, d, shape.w_std, device),
            "w_gu": _dev_weight(gen, d, 2 * f, shape.w_std, device),
            "w_down": _dev_weight(gen, f, d, shape.w_std, device),
        }
        kv_base = tuple(torch.randn((shape.n_kv_heads, shape.ctx, shape.d_head), generator=gen,
                                    device=device).to(torch.bfloat16) for _ in range(2))
        n_layers = 32
        for B, sps in ((1, (25, 40, 50)), (4, (25, 40, 50)), (16, (25, 40, 50))):
            sps = tuple(sp for sp in sps if want(f"decoder32_7b_b{B}_s{sp}"))
            if not sps:
                continue
            layers = [dec.build_layer(3, l, shape, base, kv_base, B, sps[0])[0]
                      for l in range(n_layers)]
            buf = dec.DecoderBuffers(shape, B)
            h0 = wl.to_torch(wl.decoder_hidden(3, B, d), "bf16")
            h = h0.clone()
            for sp in sps:
                for L in layers:
                    for role in dec.ROLES:
                        lin = L.lin[role]
                        lin.k = wl.k_for(lin.d_in, sp)
                    L.ws = {}

                def step():
                    h.copy_(h0)
                    dec.decoder_step(layers, h, buf, _lib.UNFUSED)
                ms = _timed_ms(step, steps, warm)
                # bytes: rotations + union rows (one traced step) + key/value cache
                nbytes = 0
                h.copy_(h0)
                traces = [{} for _ in layers]
                dec.decoder_step(layers, h, buf, _lib.UNFUSED, traces=traces)
                for L, trace in zip(layers, traces):
                    for role in dec.ROLES:
                        lin = L.lin[role]
                        nbytes += lin.Qt.numel() * 2 + _union_rows(trace[role][1]) * lin.d_out * 2
                    nbytes += B * 2 * shape.n_kv_heads * shape.ctx * shape.d_head * 2
                res[f"decoder32_7b_b{B}_s{sp}"] = _entry(B, ms, nbytes, {"layers": n_layers})
            del layers, buf
            torch.cuda.empty_cache()
        del base, kv_base
        torch.cuda.empty_cache()

    # layer slices: the four rotated linears of one layer (no attention core)
    gen = torch.Generator(device=device)
    slices = (("13b", 4, 5120, 13824, 40, 40, 0.02, "outlier", 40, (8,)),
              ("70b", 5, 8192, 28672, 64, 8, 0.01, "heavy", 50, (32, 64)))
    for name, cfg, d, f, H, Hkv, wstd, act, sp, Bs in slices:
        if not any(want(f"slice_{name}_b{B}_s{sp}") for B in Bs):
            continue
        q2 = wl.ffn_q_block(f)
        qkv_out = (H + 2 * Hkv) * 128
        gen.manual_seed(cfg)
        lins = {
            "attn_in": RotatedLinear(_dev_haar(gen, d, 1, device),
                                     _dev_weight(gen, d, qkv_out, wstd, device), "bf16",
                                     wl.k_for(d, sp), keep_w=False),
            "o_in": RotatedLinear(_dev_haar(gen, d, 1, device), _dev_weight(gen, d, d, wstd, device),
                                  "bf16", wl.k_for(d, sp), keep_w=False),
            "mlp_in": RotatedLinear(_dev_haar(gen, d, 1, device),
                                    _dev_weight(gen, d, 2 * f, wstd, device), "bf16",
                                    wl.k_for(d, sp), keep_w=False),
            "down_in": RotatedLinear(_dev_haar(gen, q2, f // q2, device),
                                     _dev_weight(gen, f, d, wstd, device), "bf16",
                                     wl.k_for(f, sp), keep_w=False),
        }
        for B in Bs:
            if not want(f"slice_{name}_b{B}_s{sp}"):
                continue

            def acts(role):
                if act == "outlier":
                    return wl.to_torch(wl.outlier_activations(cfg, 0, role, B, d, d // 100, 30.0,
                                                              "bf16"), "bf16")
                return wl.to_torch(wl.heavy_tailed_activations(cfg, 0, role, B, d, "bf16"), "bf16")
            xa, xo, xm = acts("attn_in"), acts("o_in"), acts("mlp_in")
            ya = torch.empty((B, qkv_out), dtype=torch.bfloat16, device=device)
            yo = torch.empty((B, d), dtype=torch.bfloat16, device=device)
            gu = torch.empty((B, 2 * f), dtype=torch.bfloat16, device=device)
            hh = torch.empty((B, f), dtype=torch.bfloat16, device=device)
            yd = torch.empty((B, d), dtype=torch.bfloat16, device=device)
            wss = {r: lins[r].workspace(B) for r in lins}

            def step(trace=None):
                outs = {}
                for role, xin, yout in (("attn_in", xa, ya), ("o_in", xo, yo),
                                        ("mlp_in", xm, gu)):
                    idx = None
                    if trace is not None:
                        idx = torch.empty((B, lins[role].k), dtype=torch.int32, device=device)
                        trace[role] = idx
                    lins[role].forward(xin, yout, wss[role], idx_out=idx)
                _lib.larosa_swiglu(gu, hh, B, f)
                idx = None
                if trace is not None:
                    idx = torch.empty((B, lins["down_in"].k), dtype=torch.int32, device=device)
                    trace["down_in"] = idx
                lins["down_in"].forward(hh, yd, wss["down_in"], idx_out=idx)
            ms = _timed_ms(step, steps, warm)
            trace = {}
            step(trace)
            torch.cuda.synchronize()
            nbytes = sum(lins[r].Qt.numel() * 2 + _union_rows(trace[r]) * lins[r].d_out * 2
                         for r in lins)
            rows = {r: _union_rows(trace[r]) for r in lins}
            res[f"slice_{name}_b{B}_s{sp}"] = _entry(
                B, ms, nbytes, {"union_rows": rows, "d_in": {r: lins[r].d_in for r in lins}})
        del lins
        torch.cuda.empty_cache()
    return res


def cpu_baseline(case, x, q1, wgu, q2, wd, seconds):
    """The oracle's MLP, as it stands, on the host: fold once (untimed), then
    as many single-token steps as fit in about `seconds`, once with the BLAS
    pool at every core this process may use and once at one thread. `value`
    is the all-cores rate; `cores` the threads that run used."""
    from oracle import larosa_ref as ref
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:
        threadpool_info = threadpool_limits = None
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    w1 = ref.fold(q1, wgu, "bf16")
    w2 = ref.fold(q2, wd, "bf16")

    def run(limit):
        ctx = threadpool_limits(limits=limit) if threadpool_limits else None
        if ctx is not None:
            ctx.__enter__()
        try:
            threads = (max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
                       if threadpool_info else (limit or os.cpu_count() or 1))
            ref.mlp(x, q1, w1, q2, w2, case.k1, case.k2, case.f)  # warm-up, untimed
            n = 0
            t0 = time.perf_counter()
            while True:
                ref.mlp(x, q1, w1, q2, w2, case.k1, case.k2, case.f)
                n += 1
                el = time.perf_counter() - t0
                if el >= seconds or n >= 1000:
                    break
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        return n, el, threads
    n_all, el_all, thr_all = run(affinity)
    n_one, el_one, _ = run(1)
    return {"value": round(n_all / el_all, 3), "unit": "tokens/s", "cores": thr_all,
            "kind": "oracle",
            "sample": f"{n_all} single-token steps of the same MLP (same x and weights), "
                      f"{el_all:.1f} s, BLAS pool at {thr_all} threads; fold done once "
                      f"beforehand, untimed",
            "single_thread": {"value": round(n_one / el_one, 3), "unit": "tokens/s",
                              "steps": n_one, "seconds": round(el_one, 1)},
            "os_cpu_count": os.cpu_count(), "affinity_cores": affinity}


if __name__ == "__main__":
    main()
