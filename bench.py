#!/usr/bin/env python3
"""Throughput of one GPU's share of the MoE training layer (forward + backward).

One step = one pass of the whole hot path on one batch of synthetic input:
schedule build + forward (ring gather, gate/up GEMM with SwiGLU, down GEMM,
weighted combine) + backward (dy gather, dA GEMM with SwiGLU backward and
router-weight gradient, dX GEMM with combine, router-gradient reduction,
weight-gradient GEMMs). Inputs are resident in HBM before timing starts.

Prints one JSON line. `value` is tokens/s where a token is a pre-routing
token of the GPU's share (the EP-64 share stands for 2,048 tokens per step).
Also reports the roofline of the dominant kernel among those that run alone
(per-kernel durations from HIP events the library records on each launch's
stream; dW_down, which runs beside other kernels on a side stream, gets no
rate) and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0

WORKLOAD_TEXT = {
    "ep64_share": "EP-64 one-GPU share: 16,384 routed rows (2,048 tokens x 64 ranks x top-8 / 256 experts x 4), "
                  "4 local SwiGLU experts, H=7168, I=2048, Zipf(1.2) loads 8658/3769/2317/1640, BF16, "
                  "ring 256 MiB, mini-batch 512",
    "ep64_share_mxfp8": "EP-64 one-GPU share as ep64_share in MXFP8 (E4M3 elements, E8M0 scale per 32 along K; "
                        "weights pre-quantized once, activations quantized in-kernel; weight gradients BF16), "
                        "Zipf(1.2) loads",
    "ep64_share_mxfp8_uniform": "EP-64 one-GPU share in MXFP8 as ep64_share_mxfp8, uniform loads 4 x 4,096",
    "full_layer": "single-GPU full layer: T=2048, top-8 of 256 SwiGLU experts, H=7168, I=2048, BF16",
    "stream": "fine-grained streaming share: 8 x 20,480 rows, 8 experts, H=4096, I=1024, Dirichlet(0.3), "
              "ring 128 MiB",
    "tiny": "tiny: T=64, H=128, I=64, E=8, top-2",
}


def flops_per_row(H, I):
    """Algorithmic flops per routed row, per kernel (recompute and padding not counted)."""
    return dict(gateup=4 * H * I, down=2 * H * I, dA=2 * H * I, dX=4 * H * I,
                fwd_gemms=6 * H * I, bwd_gemms=6 * H * I,           # persistent gate/up + down, dA + dX
                wgrad_gate_up=4 * H * I, wgrad_down=2 * H * I)


def _code_only(text: str) -> str:
    """Source text without // and /* */ comments and blank lines (string literals
    holding comment markers are not expected in these sources)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l)


def build_flags(build_py: str = "") -> str:
    """The compiler command-line pieces of the library's build script (its COMMON
    flag list and the source list), as text: a flag change alters the kernels."""
    build_py = build_py or os.path.join(ROOT, "mixture_experts_layer_table_amd", "build.py")
    text = open(build_py, encoding="utf-8").read()
    parts = re.findall(r"^(SOURCES|COMMON)\s*=\s*(\[.*?\])", text, re.M | re.S)
    return "\n".join(f"{k}=" + re.sub(r"\s+", "", re.sub(r"#.*", "", v)) for k, v in parts)


def source_digest(csrc: str = "", build_py: str = "") -> str:
    """Digest of everything that decides the kernels' code and launches: the HIP
    files, the headers they include, the host sources (plan, streams, timing:
    slot counts, workspace layout, launch shapes) and the build flags, comments
    excluded, so that a comment edit does not retire the counters."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "mixture_experts_layer_table_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")) +
                    glob.glob(os.path.join(csrc, "*.cpp"))):
        h.update(_code_only(open(p, encoding="utf-8").read()).encode())
    h.update(build_flags(build_py).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed PMC summary, or None when
    the summary is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_digest") != source_digest():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(inp, tokens_per_step, seconds):
    """The oracle as it stands, on a bounded sample of routed rows of the same
    workload: forward and backward of each sampled row, extrapolated to the step
    (with the MXFP8 fake-quant in MXFP8 mode)."""
    import numpy as np
    from oracle import layer as L
    from oracle import mxfp8 as M
    fq = M.fake_quant if inp.cfg.precision == "mxfp8" else None
    try:
        from threadpoolctl import threadpool_info
        cores = sum(i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        cores = 1
    cfg = inp.cfg
    f = L.bf16_bits_to_f64
    flat = inp.topk_ids.reshape(-1)
    wflat = inp.topk_w.reshape(-1).astype(np.float64)
    done, busy, chunk = 0, 0.0, 64
    for e in range(cfg.E):                       # every row costs the same: any rows are a fair sample
        rows_e = np.nonzero(flat == e)[0]
        if rows_e.size == 0:
            continue
        Wg, Wu, Wd = f(inp.w_gate[e]), f(inp.w_up[e]), f(inp.w_down[e])   # decoded once, untimed
        for c0 in range(0, rows_e.size, chunk):
            rows = rows_e[c0: c0 + chunk]
            tok = rows // cfg.k
            t = time.perf_counter()
            xe, dye = f(inp.x[tok]), f(inp.dy[tok])
            L.expert_forward(xe, Wg, Wu, Wd, fq)
            L.expert_backward(xe, dye, wflat[rows][:, None], Wg, Wu, Wd, fq)
            busy += time.perf_counter() - t
            done += rows.size
            if busy >= seconds:
                break
        if busy >= seconds:
            break
    el = busy
    step_s = el * cfg.R / max(done, 1)
    return dict(value=tokens_per_step / step_s, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{done} of {cfg.R} routed rows (forward + backward, fp64 numpy) in {el:.1f} s, "
                       f"extrapolated linearly to the step")


def library_gemm_rates(cfg, steps):
    """hipBLASLt bf16 rates (torch.matmul, fp32 accumulation) for the dense GEMMs
    with the shapes of the layer's grouped GEMMs over all R routed rows: gate/up
    [R,H]x[H,2I], down [R,I]x[I,H], dA [R,H]x[H,I], dX [R,2I]x[2I,H]."""
    import torch
    torch.backends.cuda.preferred_blas_library("hipblaslt")
    R, H, I = cfg.R, cfg.H, cfg.I
    out = dict(kind="library_gemm", library="hipblaslt via torch.matmul", dtype="bf16", rows=R, shapes={})
    for name, (m, k, n) in dict(gateup=(R, H, 2 * I), down=(R, I, H), dA=(R, H, I), dX=(R, 2 * I, H)).items():
        a = torch.randn(m, k, device="cuda:0").to(torch.bfloat16)
        b = torch.randn(k, n, device="cuda:0").to(torch.bfloat16)
        for _ in range(3):
            c = a @ b
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out["shapes"][name] = dict(m=m, k=k, n=n, ms=round(ms, 4), tflops=round(2 * m * k * n / ms / 1e9, 1))
        del a, b, c
    return out


def sweep(args, cfg, base, n_cu, ids, tw, x, dy, wg, wu, wd, w_fwd, w_bwd, dev):
    """Step time over mini-batch rows x ring size; no knob changes a result bit, so the
    outputs of every point are compared with the first point's, byte for byte."""
    import numpy as np
    import torch

    import mixture_experts_layer_table_amd as mok
    row_bytes = 2 * cfg.H if base.precision == mok.MOK_BF16 else cfg.H + cfg.H // 32
    pick = mok.autosize_config(base, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, n_cu)
    macro_rows = cfg.k * (cfg.T if cfg.macrobatch_tokens in (0,) or cfg.macrobatch_tokens >= cfg.T
                          else cfg.macrobatch_tokens)
    points = []
    for mb in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
        if mb > max(2 * macro_rows, 256):
            continue
        for ring in sorted({2 * mb * row_bytes, max(cfg.ring_bytes, 2 * mb * row_bytes)}):
            points.append((mb, ring))
    if (pick.minibatch_rows, pick.ring_bytes) not in points:
        points.append((pick.minibatch_rows, pick.ring_bytes))
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    grads = dict(dx=torch.empty_like(x), dw_gate=torch.empty_like(wg), dw_up=torch.empty_like(wu),
                 dw_down=torch.empty_like(wd), dtopk_w=torch.empty_like(tw))
    first = None
    results = []
    for mb, ring in points:
        c = dataclasses.replace(base, minibatch_rows=mb, ring_bytes=ring)
        ws = mok.get_workspace(c, device=dev, num_local_tokens=cfg.T, hidden_size=cfg.H,
                               intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
        sched = torch.empty(ws.schedule_bytes, dtype=torch.uint8, device=dev)
        ctx = torch.empty(ws.fwd_ctx_bytes, dtype=torch.uint8, device=dev)

        def step():
            mok.build_schedule(ws, ids, sched)
            mok.forward(ws, sched, x, tw, w_fwd, out=out, fwd_ctx=ctx)
            mok.backward(ws, sched, ctx, x, tw, w_bwd, dy, grads=grads)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        status = int(sched[:4].cpu().numpy().view(np.uint32)[0])
        digest = [out.clone()] + [grads[n].clone() for n in ("dx", "dw_gate", "dw_up", "dw_down", "dtopk_w")]
        if first is None:
            first = digest
        same = all(torch.equal(a.view(torch.uint8) if a.dtype != torch.float32 else a.view(torch.int32),
                               b.view(torch.uint8) if b.dtype != torch.float32 else b.view(torch.int32))
                   for a, b in zip(digest, first))
        ms = e0.elapsed_time(e1) / args.steps
        n_slots = ring // (mb * row_bytes)
        rec = dict(sweep=args.workload, minibatch_rows=mb, ring_bytes=ring, ring_slots=n_slots,
                   rows_per_round=min(n_slots * mb, cfg.R), ms_per_step=round(ms, 4),
                   tokens_per_s=round(cfg.tokens_per_step / (ms * 1e-3), 1), status=status,
                   bitwise_equal_to_first=bool(same),
                   two_wave_pick=(mb, ring) == (pick.minibatch_rows, pick.ring_bytes))
        results.append(rec)
        print(json.dumps(rec), flush=True)
        del ws, sched, ctx
        torch.cuda.empty_cache()
    best = min(results, key=lambda r: r["ms_per_step"])
    pick_rec = next(r for r in results if r["two_wave_pick"])
    print(json.dumps(dict(sweep_summary=args.workload, n_cu=n_cu,
                          pick=dict(minibatch_rows=pick.minibatch_rows, ring_bytes=pick.ring_bytes,
                                    ms_per_step=pick_rec["ms_per_step"]),
                          best=dict(minibatch_rows=best["minibatch_rows"], ring_bytes=best["ring_bytes"],
                                    ms_per_step=best["ms_per_step"]),
                          pick_over_best=round(pick_rec["ms_per_step"] / best["ms_per_step"], 4),
                          all_bitwise_equal=all(r["bitwise_equal_to_first"] for r in results),
                          all_status_clear=all(r["status"] == 0 for r in results))), flush=True)


TRACE_KERNELS = {0: "fwd_gemms", 1: "bwd_gemms", 2: "wgrad_gate_up", 3: "wgrad_down", 4: "other"}


def item_trace_summary(rec, cfg):
    """Where the compute units' time goes in each traced GEMM kernel, from the
    per-item records (100 MHz clock): per launch, each workgroup's span from the
    launch's first record to its last is split into claim and input wait, K
    loop, epilogue (stores and publication), idle before its first item and
    idle after its last; shares are over workgroups x launch span, averaged
    over launches of the same kernel. A persistent workgroup takes its next
    ticket during the current item's epilogue, so an item's claim time counts
    from the later of its claim record and the end of the workgroup's
    previous item. Also microseconds per item and per K step for each item
    class whose K is fixed (segment GEMMs)."""
    import numpy as np
    H, I = cfg.H, cfg.I
    ksteps = {(0, 1): H // 32, (0, 2): I // 32, (1, 1): H // 32, (1, 2): 2 * I // 32}
    out = {}
    for kern in sorted(set(rec["kernel"].tolist())):
        rk = rec[rec["kernel"] == kern]
        shares, per_class = [], {}
        for launch in sorted(set(rk["launch"].tolist())):
            r = rk[rk["launch"] == launch].copy()
            t0, t1 = int(r["t_claim"].min()), int(r["t_end"].max())
            # claim start: not before the workgroup's previous item ended
            for wg in set(r["workgroup"].tolist()):
                idx = np.flatnonzero(r["workgroup"] == wg)
                idx = idx[np.argsort(r["t_start"][idx], kind="stable")]
                prev_end = np.concatenate([[0], r["t_end"][idx][:-1]])
                r["t_claim"][idx] = np.maximum(r["t_claim"][idx], prev_end)
            span = max(t1 - t0, 1)
            wgs = sorted(set(r["workgroup"].tolist()))
            tot = dict(claim=0, kloop=0, epilogue=0, idle_start=0, idle_end=0)
            for wg in wgs:
                w = r[r["workgroup"] == wg]
                tot["claim"] += int((w["t_start"] - w["t_claim"]).sum())
                tot["kloop"] += int((w["t_kloop"] - w["t_start"]).sum())
                tot["epilogue"] += int((w["t_end"] - w["t_kloop"]).sum())
                tot["idle_start"] += int(w["t_claim"].min()) - t0
                tot["idle_end"] += t1 - int(w["t_end"].max())
            denom = span * len(wgs)
            shares.append({k: v / denom for k, v in tot.items()} | dict(span_us=span / 100.0, workgroups=len(wgs)))
            for cls in sorted(set(r["item_class"].tolist())):
                c = r[r["item_class"] == cls]
                d = per_class.setdefault(int(cls), dict(items=0, kloop=0, epi=0, claim=0))
                d["items"] += len(c)
                d["kloop"] += int((c["t_kloop"] - c["t_start"]).sum())
                d["epi"] += int((c["t_end"] - c["t_kloop"]).sum())
                d["claim"] += int((c["t_start"] - c["t_claim"]).sum())
        avg = {k: round(float(np.mean([s[k] for s in shares])), 4) for k in shares[0]}
        avg["launches"] = len(shares)
        classes = {}
        for cls, d in per_class.items():
            n = max(d["items"], 1)
            e = dict(items_per_launch=round(d["items"] / len(shares), 1), kloop_us=round(d["kloop"] / n / 100.0, 2),
                     epilogue_us=round(d["epi"] / n / 100.0, 2), claim_us=round(d["claim"] / n / 100.0, 2))
            if (kern, cls) in ksteps:
                e["us_per_kstep"] = round(d["kloop"] / n / 100.0 / ksteps[(kern, cls)], 3)
            classes[cls] = e
        out[TRACE_KERNELS.get(kern, str(kern))] = dict(shares=avg, classes=classes)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ep64_share", choices=list(WORKLOAD_TEXT))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--minibatch-rows", type=int, default=0,
                    help="override the workload's mini-batch size (results do not depend on it)")
    ap.add_argument("--separate-launches", action="store_true",
                    help="one launch per grouped GEMM instead of the persistent pair kernels (per-GEMM timing)")
    ap.add_argument("--item-trace", action="store_true",
                    help="record the per-item trace of the GEMM kernels over --steps steps and print its summary")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the layer, run a plain device-to-device copy of this many MiB "
                         "(calibrates the HBM byte counters against a kernel of known traffic)")
    ap.add_argument("--autosize", action="store_true",
                    help="size the mini-batch by the two-wave rule (mok_config_autosize) instead of the "
                         "workload's setting")
    ap.add_argument("--mx-wgrad", action="store_true",
                    help="MXFP8 workloads: weight gradients on the block-scaled MFMA too (MOK_MXFP8_WGRAD)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of one bench line, time the step over a grid of mini-batch sizes and ring "
                         "sizes (plus the two-wave pick) and print one JSON line per point, then a summary")
    ap.add_argument("--library-gemm", action="store_true",
                    help="instead of the layer, time the vendor library's dense bf16 GEMM (torch.matmul on "
                         "hipBLASLt) at the workload's four grouped-GEMM shapes taken as single dense GEMMs: "
                         "a reference rate for the grouped GEMMs on this GPU, not part of the layer")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_layer_table_amd as mok
    import synth

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_probe_bytes=n, launches=args.steps)), flush=True)
        return

    if args.library_gemm:
        print(json.dumps(library_gemm_rates(synth.CONFIGS[args.workload], args.steps)), flush=True)
        return

    cfg = synth.CONFIGS[args.workload]
    if args.minibatch_rows:
        cfg = dataclasses.replace(cfg, minibatch_rows=args.minibatch_rows)
    dev = "cuda:0"
    inp = synth.make_inputs(cfg)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    ids = torch.from_numpy(inp.topk_ids).to(dev)
    tw = torch.from_numpy(inp.topk_w).to(dev)
    x, dy = bf16(inp.x), bf16(inp.dy)
    wg, wu, wd = bf16(inp.w_gate), bf16(inp.w_up), bf16(inp.w_down)
    mx = cfg.precision == "mxfp8"
    quant_ms = None
    if mx:   # weights quantized once per step of a training loop's weight update, outside the layer's time
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record()
        qw = mok.MXFP8Weights(wg, wu, wd)
        q1.record()
        torch.cuda.synchronize()
        quant_ms = q0.elapsed_time(q1)
        w_fwd, w_bwd = qw.fwd, qw.bwd
    else:
        w_fwd = w_bwd = mok.weights_bf16(wg, wu, wd)
    config = mok.MoKConfig(minibatch_rows=cfg.minibatch_rows, macrobatch_tokens=cfg.macrobatch_tokens,
                           ring_bytes=cfg.ring_bytes,
                           precision=(mok.MOK_MXFP8_WGRAD if args.mx_wgrad else mok.MOK_MXFP8) if mx else mok.MOK_BF16,
                           debug_flags=mok.MOK_DEBUG_SEPARATE_LAUNCHES if args.separate_launches else 0)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    if args.autosize:
        config = mok.autosize_config(config, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, n_cu)
        cfg = dataclasses.replace(cfg, minibatch_rows=config.minibatch_rows, ring_bytes=config.ring_bytes)
    if args.sweep:
        sweep(args, cfg, config, n_cu, ids, tw, x, dy, wg, wu, wd, w_fwd, w_bwd, dev)
        return
    ws = mok.get_workspace(config, device=dev, num_local_tokens=cfg.T, hidden_size=cfg.H,
                           intermediate_size=cfg.I, num_experts=cfg.E, topk=cfg.k)
    sched = torch.empty(ws.schedule_bytes, dtype=torch.uint8, device=dev)
    ctx = torch.empty(ws.fwd_ctx_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev)
    grads = dict(dx=torch.empty_like(x), dw_gate=torch.empty_like(wg), dw_up=torch.empty_like(wu),
                 dw_down=torch.empty_like(wd), dtopk_w=torch.empty_like(tw))

    def step():
        mok.build_schedule(ws, ids, sched)
        mok.forward(ws, sched, x, tw, w_fwd, out=out, fwd_ctx=ctx)
        mok.backward(ws, sched, ctx, x, tw, w_bwd, dy, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(sched[:4].cpu().numpy().view(np.uint32)[0]) == 0, "schedule status word set"
    if args.item_trace:
        mok._check(mok.mok_item_trace_enable(1), "mok_item_trace_enable")
        for _ in range(args.steps):
            step()
        rec, n = mok.item_trace_read()
        mok._check(mok.mok_item_trace_enable(0), "mok_item_trace_enable")
        print(json.dumps(dict(item_trace=args.workload, steps=args.steps, records=int(n),
                              summary=item_trace_summary(rec, cfg))), flush=True)
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert int(sched[:4].cpu().numpy().view(np.uint32)[0]) == 0, "status word set during the timed steps"
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps

    # per-kernel durations: HIP events recorded by the library around each launch
    nprof = min(args.steps, 10)
    mok._check(mok.mok_kernel_timing_enable(1), "timing")
    for _ in range(nprof):
        step()
    torch.cuda.synchronize()
    ktimes = mok.kernel_times()
    R, H, I = cfg.R, cfg.H, cfg.I
    fpr = flops_per_row(H, I)
    kernels = {}
    for name, (launches, total_ms, max_ms) in ktimes.items():
        avg = total_ms / launches
        entry = dict(launches_per_step=launches / nprof, avg_ms=round(avg, 5), ms_per_step=round(total_ms / nprof, 4))
        if name in fpr:
            fl = fpr[name] * R * nprof / launches
            entry["tflops"] = round(fl / (avg * 1e-3) / 1e12, 1)
        if name in ("gather", "gather_dy"):
            by = (2 * cfg.T * H + 2 * R * H + 4 * R) * nprof / launches   # unique reads + writes
            entry["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
        if name in ("combine", "combine_dx"):   # k > 1: staged rows read, token rows written
            by = (2 * R * H + 2 * cfg.T * H + 8 * R) * nprof / launches
            entry["gbs"] = round(by / (avg * 1e-3) / 1e9, 1)
        kernels[name] = entry
    fp8_kernels = ("gateup", "down", "dA", "dX", "fwd_gemms", "bwd_gemms") if mx else ()
    if mx and args.mx_wgrad:
        fp8_kernels += ("wgrad_gate_up", "wgrad_down")
    # With BF16 weight gradients, dW_down runs on a side stream beside the last
    # dgrad GEMMs and dW_gate | dW_up: its span includes time it shares with
    # them, so it gets no rate, and the roofline and the GEMM utilisation use
    # the kernels that run alone.
    side = () if (mx and args.mx_wgrad) else ("wgrad_down",)
    for n in kernels:
        if n in fpr:
            peak = PEAK_FP8_TFLOPS if n in fp8_kernels else PEAK_BF16_TFLOPS
            kernels[n]["mfma_dtype"] = "mxfp8" if n in fp8_kernels else "bf16"
            if n in side:
                kernels[n]["beside"] = True
                del kernels[n]["tflops"]
            else:
                kernels[n]["frac_of_peak"] = round(kernels[n]["tflops"] / peak, 4)
    alone = [n for n in kernels if n in fpr and n not in side]
    dominant = max(alone, key=lambda n: kernels[n]["ms_per_step"])
    dk = kernels[dominant]
    ach = dk["tflops"]
    dpeak = PEAK_FP8_TFLOPS if dominant in fp8_kernels else PEAK_BF16_TFLOPS
    roofline = dict(bound="mfma", kernel=dominant, achieved=ach, peak=dpeak, unit="TFLOP/s",
                    frac=round(ach / dpeak, 4),
                    traffic=read_traffic(args.workload, dominant),
                    flops_per_launch=fpr[dominant] * R * nprof / ktimes[dominant][0],
                    avg_launch_ms=dk["avg_ms"],
                    timing_source=f"HIP events the library records around each launch on the launch's own "
                                  f"stream, over {nprof} steps after the timed region (the rocprofv3 kernel "
                                  f"trace of the same command is the cross-check)")

    total_flops = 18 * R * H * I
    # time at the MFMA peaks: fwd + dA + dX (12 RHI) on the fp8 peak in MXFP8 mode, the rest bf16
    peak_time_s = ((12 * R * H * I) / (PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS)
                   + (6 * R * H * I) / (PEAK_FP8_TFLOPS if mx and args.mx_wgrad else PEAK_BF16_TFLOPS)) / 1e12
    tokens = cfg.tokens_per_step
    value = tokens / (ms_per_step * 1e-3)
    sched_ms = kernels.get("schedule", {}).get("ms_per_step", 0.0)
    res = dict(
        metric="MoE layer fwd+bwd tokens/s on 1 GPU; grouped-GEMM MFMA util % of peak",
        value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="mxfp8" if mx else "bf16", data="synthetic",
        config=dict(workload=f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", T=cfg.T, H=H, I=I, E=cfg.E,
                    k=cfg.k, routed_rows=R, tokens_per_step=tokens, minibatch_rows=cfg.minibatch_rows,
                    macrobatch_tokens=cfg.macrobatch_tokens, ring_bytes=cfg.ring_bytes),
        rows_per_s=round(R / (ms_per_step * 1e-3), 1),
        tflops=round(total_flops / (ms_per_step * 1e-3) / 1e12, 1),
        mfma_util=round(peak_time_s / (ms_per_step * 1e-3), 4),
        # the grouped GEMMs that run alone: their flops at peak over their summed kernel time
        gemm_mfma_util=round(sum(fpr[n] * R * (PEAK_FP8_TFLOPS if n in fp8_kernels else PEAK_BF16_TFLOPS) ** -1
                                 for n in alone) / 1e12 / (sum(kernels[n]["ms_per_step"] for n in alone) * 1e-3), 4),
        schedule_share=round(sched_ms / ms_per_step, 4) if sched_ms else None,
        weight_quantize_ms=round(quant_ms, 4) if quant_ms is not None else None,
        roofline=roofline, kernels=kernels, source_digest=source_digest(),
        device=torch.cuda.get_device_name(0),
    )
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, tokens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
