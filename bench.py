"""Benchmark of the MoE-layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens: one moe_layer
call (routing with the layout's chunk histogram in the same launch, the layout, gate/up
reading the token rows through row_token, down, combine; the capacity selection too when
the workload has a cap).  With --router the step is the staged sequence below with
moe_router in front.  Inputs and the packed expert weights are resident in HBM before
timing starts.

Prints one JSON line: whole-step throughput in tokens/s, the roofline of the dominant
kernel (per-launch algorithmic bytes or flops over its HIP-event-timed duration on the
launch stream), and the CPU oracle timed on a bounded sample of the same workload.

Two passes over the same steps: the timed pass (the `value`) records no events -- a timing
event between kernels costs about 10 us of GPU time on this stack -- and a second pass of
the same number of steps issues the layer's kernel sequence through the staged entry
points,
  moe_route -> moe_dispatch (layout only) -> moe_expert_gate_up_gather -> moe_expert_down
  -> moe_combine,
with an event before and after every stage, on the launch stream, for the per-stage
durations and the dominant kernel's roofline.  (There the layout counts its chunk
histogram in a launch of its own: moe_route hands none over.)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec on 1 MI355X; % bf16 MFMA peak (GEMM), % HBM peak (dispatch)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, GB/s
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}  # dense MFMA bf16, fp8; fp32 vector
DEFAULT_WORKLOAD = "dsv3_prefill"  # the largest single-GPU workload
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its steady clock only after some 50-100 ms of back-to-back steps (a
    # 0.46 ms step runs at ~0.50 ms over the first 20): the warm-up runs at least
    # --warmup steps and at least --warmup-seconds of them, whichever is longer
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-seconds", type=float, default=0.5)
    ap.add_argument("--config", default=DEFAULT_WORKLOAD)
    ap.add_argument("--router", action="store_true",
                    help="route from the hidden states: router GEMM x W_r^T + selection "
                         "(moe_router; DeepSeek-V3-style 8/4 expert groups when E = 256) instead "
                         "of moe_route on given logits")
    ap.add_argument("--chunk-tokens", type=int, default=0,
                    help="also time moe_layer and moe_layer_chunked with chunks of this many "
                         "tokens (layouts on an auxiliary stream); reported under 'layer_calls'")
    ap.add_argument("--shared-I", type=int, default=0,
                    help="with --chunk-tokens: a shared expert of this intermediate width")
    ap.add_argument("--backward", action="store_true",
                    help="also time moe_layer_backward (saved routing, expert outputs and g|u of the "
                         "timed forward, bf16 upstream gradient); reported under 'backward'")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="cold-cache pass: a scratch write of this many MiB before every step "
                         "(0: no cold-cache pass); reported under 'cold_cache'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference "
                         "for scaling HBM byte counters)")
    return ap.parse_args()


def algorithmic(wl, N, E_hit, router=False):
    """Per-stage algorithmic HBM bytes and flops (decimal units): every input read once and
    every output written once.  FP8 weights and the FP8 intermediate count one byte per
    element plus one scale byte per 32; the FP8 gate/up stage starts from the bf16 token
    rows (its per-row quantisation is part of the stage)."""
    b = 4 if wl.dtype == "f32" else 2                       # activations
    wb = 1 + 1 / 32 if wl.dtype == "fp8" else b             # weights
    ab = 1 + 1 / 32 if wl.dtype == "fp8" else b             # intermediate a
    T, H, E, k, I = wl.T, wl.H, wl.E, wl.k, wl.I
    return {
        # with the router: x and W_r in (bf16), ids/weights/keep out; else logits in
        "route": (dict(bytes=T * H * 2 + E * H * 2 + T * k * 9, flops=2 * T * H * E) if router
                  else dict(bytes=T * E * 4 + T * k * 9, flops=0)),
        # ids (+ keep) in; counts, offsets, row_token, slot_to_row out
        "dispatch": dict(bytes=T * k * 5 + N * 4 + T * k * 4 + E * 8, flops=0),
        # weights of the experts hit, the token rows x (once) and row_token in; a out
        "gate_up": dict(bytes=E_hit * 2 * H * I * wb + T * H * b + N * 4 + N * I * ab,
                        flops=4 * N * H * I),
        "down": dict(bytes=E_hit * I * H * wb + N * I * ab + N * H * b, flops=2 * N * H * I),
        "combine": dict(bytes=N * H * b + T * k * 8 + T * H * b, flops=0),
    }


def roofline_of(stage, alg, sec, dtype):
    a = alg[stage]
    if stage == "route":
        dtype = "bf16"  # the router GEMM runs in bf16 whatever the expert weights
    t_hbm = a["bytes"] / (PEAK_HBM_GBS * 1e9)
    t_mfma = a["flops"] / (PEAK_TFLOPS[dtype] * 1e12) if a["flops"] else 0.0
    if t_mfma > t_hbm:
        ach = a["flops"] / sec / 1e12
        return dict(bound="alu" if dtype == "f32" else "mfma", achieved=round(ach, 2),
                    peak=PEAK_TFLOPS[dtype], unit="TFLOP/s", frac=round(ach / PEAK_TFLOPS[dtype], 4))
    ach = a["bytes"] / sec / 1e9
    return dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                frac=round(ach / PEAK_HBM_GBS, 4))


def kernel_source_hash(csrc=None, files=None):
    """Hash of the kernel sources (all of them, or the named files) with comments and blank
    lines removed (a comment edit leaves the kernels, and so the recorded counters, valid)."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "expert_ffn_moe_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines())
        h.update(f.encode() + b"\0" + "\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current sources of the stage's kernels (the record's kernel_files; all sources if it
    names none), else None."""
    path = os.path.join(PROFILES, f"traffic_{stage}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources") != kernel_source_hash(files=rec.get("kernel_files")):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, inp, target_s, wr=None, groups=(1, 1)):
    """The oracle (as it stands) on a bounded sample: routing, capacity and layout over all
    T tokens, the FFN and combine over a sample of tokens; scaled to tokens/s."""
    import numpy as np

    import oracle
    import synth

    import torch

    # every core this process may use, capped by the thread count the environment sets
    # (OMP_NUM_THREADS: a host shared between GPUs gives each its share)
    avail = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(avail, int(env)) if env.isdigit() and int(env) > 0 else avail
    model, ncpu = host_cpu()
    host = {n: (synth.bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy())
            for n, t in inp.items()}
    fp8 = wl.dtype == "fp8"
    if fp8:  # weight quantisation is the one-time packing step: outside the timed part
        wq = [oracle.quant_weights(host[n]) for n in ("w_gate", "w_up", "w_down")]
    t0 = time.perf_counter()
    if wr is not None:  # router front-end: fp64 logits from x and W_r, then the selection
        lg = oracle.router_logits(host["x"], synth.bf16_bits(wr)).astype(np.float32)
        ids, w = oracle.route_grouped(lg, wl.k, groups[0], groups[1], wl.renormalize)
    else:
        ids, w = oracle.route(host["logits"], wl.k, wl.renormalize)
    keep = oracle.capacity(ids, w, wl.E, wl.capacity)
    lay = oracle.layout(ids, keep, wl.E)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(0)

    def ffn_for(tokens):
        rows = lay["slot_to_row"][tokens].ravel()
        rows = np.sort(rows[rows >= 0])
        rexp = (np.searchsorted(lay["offsets"], rows, side="right") - 1).astype(np.int32)
        xrows = host["x"][lay["row_token"][rows]]
        t1 = time.perf_counter()
        if fp8:
            xq, xs = oracle.quant_rows(xrows)
            yp = oracle.ffn_rows_fp8(xq, xs, rexp, *wq, nthreads=threads)
        else:
            yp = oracle.ffn_rows(xrows, rexp, host["w_gate"], host["w_up"], host["w_down"],
                                 nthreads=threads)
        pos = {int(r): i for i, r in enumerate(rows)}
        s2r = np.array([[pos.get(int(r), -1) for r in lay["slot_to_row"][t]] for t in tokens], np.int32)
        oracle.combine(np.arange(len(tokens), dtype=np.int32), w[tokens], s2r, yp)
        return time.perf_counter() - t1

    # calibrate on a few tokens, then size the sample to about target_s of CPU time
    n0 = min(wl.T, 8)
    t_small = ffn_for(rng.choice(wl.T, n0, replace=False))
    per_tok = max(t_small / n0, 1e-6)
    n = int(min(wl.T, max(n0, target_s / per_tok)))
    tokens = rng.choice(wl.T, n, replace=False)
    t_ffn = ffn_for(tokens)
    total = t_route + t_ffn * wl.T / n
    return dict(value=round(wl.T / total, 2), unit="tokens/s", cores=threads, kind="oracle",
                cpu_model=model, host_logical_cpus=ncpu, affinity_cpus=avail,
                sample=f"routing+capacity+layout over all {wl.T} tokens ({t_route:.2f} s); FFN+combine "
                       f"over {n} random tokens ({t_ffn:.2f} s), scaled to {wl.T} tokens")


def warm_up(fn, min_steps, min_seconds):
    """Runs fn at least min_steps times and for at least min_seconds of wall time (the GPU
    clock settles only after some 50-100 ms of back-to-back work); returns the count."""
    import torch

    n = 0
    t0 = time.perf_counter()
    while n < min_steps or time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
        if n % 8 == 0 or n >= min_steps:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def host_cpu():
    """CPU model and logical CPU count of the host, from /proc/cpuinfo."""
    model, n = "unknown", 0
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                n += 1
    except OSError:
        pass
    return model, n


def time_layer_calls(args, moe, p, wl, inp, pgu, pd, dev):
    """ms per call of moe_layer and of moe_layer_chunked (with an auxiliary stream, and with
    a shared expert if asked), every buffer allocated before timing."""
    import torch

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return round((time.perf_counter() - t0) / args.steps * 1e3, 4)

    y = torch.empty(wl.T, wl.H, dtype=p.torch_dtype, device=dev)
    ws_l = moe.workspace(p, moe.OP_LAYER, dev)
    res = {"layer_ms": timed(lambda: moe.layer(p, inp["x"], inp["logits"], pgu, pd, out=y,
                                                ws=ws_l))}
    shared = None
    if args.shared_I > 0:
        g = torch.Generator(device=dev)
        g.manual_seed(12345)
        I = args.shared_I
        sw = [(torch.randn(1, wl.H, I, generator=g, device=dev) / wl.H ** 0.5).to(torch.bfloat16),
              (torch.randn(1, wl.H, I, generator=g, device=dev) / wl.H ** 0.5).to(torch.bfloat16),
              (torch.randn(1, I, wl.H, generator=g, device=dev) / I ** 0.5).to(torch.bfloat16)]
        spgu, spd = moe.pack_weights(moe.shared_problem(p, I), *sw)
        shared = (I, spgu, spd)
    aux = torch.cuda.Stream()
    c = p.c()
    import ctypes
    need = int(moe.lib.moe_layer_chunked_workspace_bytes(ctypes.byref(c), args.chunk_tokens,
                                                         args.shared_I))
    ws_c = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    res["chunk_tokens"] = args.chunk_tokens
    res["shared_I"] = args.shared_I
    res["chunked_ms"] = timed(lambda: moe.layer_chunked(p, inp["x"], inp["logits"], pgu, pd,
                                                        args.chunk_tokens, shared=shared,
                                                        aux_stream=aux, out=y, ws=ws_c))
    res["chunked_one_stream_ms"] = timed(lambda: moe.layer_chunked(
        p, inp["x"], inp["logits"], pgu, pd, args.chunk_tokens, shared=shared, out=y, ws=ws_c))
    res["workspace_bytes"] = {"layer": int(ws_l.numel()), "chunked": need}
    return res


def time_backward(args, moe, p, wl, inp, pgu, pd, routing, disp, yp, dev):
    """ms per moe_layer_backward call on the last forward's routing and expert outputs, and
    the matrix-core rate over its GEMM flops (data gradients: da 2NHI, dxp 4NHI; weight
    gradients 2NHI + 4NHI; the g|u recompute 4NHI more when the forward did not save them).
    Timed twice: with the pre-activations saved by the forward's gate/up
    (moe_expert_gate_up_gather_gu), and recomputing them; plus what saving them adds to the
    forward's gate/up."""
    import torch

    if wl.dtype != "bf16":
        return {"skipped": "the backward pass takes bf16 problems"}
    pbgu, pbd = moe.pack_weights_backward(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    dy = torch.randn(wl.T, wl.H, generator=g, device=dev).to(torch.bfloat16)
    saved = dict(topk_ids=routing[0], topk_w=routing[1], offsets=disp["offsets"],
                 row_token=disp["row_token"], slot_to_row=disp["slot_to_row"])
    ws = moe.workspace(p, moe.OP_BACKWARD, dev)
    a_buf, gu = moe.expert_gate_up_gather_gu(p, inp["x"], disp["row_token"], disp["offsets"], pgu)

    def timed(fn, n):
        for _ in range(max(2, args.warmup // 4)):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    n = max(3, args.steps // 2)
    common = (p, inp["x"], inp["logits"], pgu, pd, pbgu, pbd, saved, dy)
    sec = timed(lambda: moe.layer_backward(*common, yp=yp, ws=ws, gu=gu), n)
    sec_rc = timed(lambda: moe.layer_backward(*common, yp=yp, ws=ws), n)
    m = max(5, args.steps)
    gu_fwd = timed(lambda: moe.expert_gate_up_gather_gu(p, inp["x"], disp["row_token"],
                                                        disp["offsets"], pgu, out=a_buf, gu=gu), m)
    plain_fwd = timed(lambda: moe.expert_gate_up_gather(p, inp["x"], disp["row_token"],
                                                        disp["offsets"], pgu, out=a_buf), m)
    N = int(disp["offsets"][-1].item())
    flops = 12 * N * wl.H * wl.I
    flops_rc = 16 * N * wl.H * wl.I
    peak = PEAK_TFLOPS["bf16"]
    return {"ms": round(sec * 1e3, 4), "calls": n, "with": "the forward's saved g|u",
            "gemm_tflops": round(flops / sec / 1e12, 1),
            "frac_bf16_peak": round(flops / sec / 1e12 / peak, 4),
            "ms_recompute_gu": round(sec_rc * 1e3, 4),
            "frac_bf16_peak_recompute_gu": round(flops_rc / sec_rc / 1e12 / peak, 4),
            "forward_gate_up_us": {"plain": round(plain_fwd * 1e6, 1),
                                   "saving_gu": round(gu_fwd * 1e6, 1)},
            "workspace_bytes": int(ws.numel())}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "launches": 3}), flush=True)
        return

    import expert_ffn_moe_amd as moe
    import synth

    wl = synth.WORKLOADS[args.config]
    p = moe.Problem.of(wl)
    dev = "cuda"
    inp = synth.make_inputs(wl, dev)
    pgu, pd = moe.pack_weights(p, inp["w_gate"], inp["w_up"], inp["w_down"])
    torch.cuda.synchronize()
    tk = wl.T * wl.k
    dt = p.torch_dtype
    # every buffer allocated once, outside the timed region
    ws = {op: moe.workspace(p, op, dev)
          for op in (moe.OP_ROUTE, moe.OP_DISPATCH, moe.OP_FFN, moe.OP_ROUTER)}
    routing = (torch.empty(wl.T, wl.k, dtype=torch.int32, device=dev),
               torch.empty(wl.T, wl.k, dtype=torch.float32, device=dev),
               torch.empty(wl.T, wl.k, dtype=torch.uint8, device=dev))
    disp = dict(counts=torch.empty(wl.E, dtype=torch.int32, device=dev),
                offsets=torch.empty(wl.E + 1, dtype=torch.int32, device=dev),
                row_token=torch.empty(tk, dtype=torch.int32, device=dev),
                slot_to_row=torch.empty(wl.T, wl.k, dtype=torch.int32, device=dev), xp=None)
    a_shape, a_dtype = p.a_shape()
    a = torch.empty(a_shape, dtype=a_dtype, device=dev)
    yp = torch.empty(tk, wl.H, dtype=dt, device=dev)
    y = torch.empty(wl.T, wl.H, dtype=dt, device=dev)
    stages = ["route", "dispatch", "gate_up", "down", "combine"]
    groups = (8, 4) if wl.E == 256 else (1, 1)
    wr = synth.make_router_weights(wl, dev) if args.router else None

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        if wr is not None:
            ids, w, keep, _ = moe.router(p, inp["x"], wr, *groups, out=routing,
                                         ws=ws[moe.OP_ROUTER])
        else:
            ids, w, keep = moe.route(p, inp["logits"], out=routing, ws=ws[moe.OP_ROUTE])
        mark(1)
        moe.dispatch(p, inp["x"], ids, keep if wl.capacity > 0 else None, out=disp,
                     ws=ws[moe.OP_DISPATCH], rows=False)
        mark(2)
        moe.expert_gate_up_gather(p, inp["x"], disp["row_token"], disp["offsets"], pgu, out=a,
                                  ws=ws[moe.OP_FFN] if p.fp8 else None)
        mark(3)
        moe.expert_down(p, a, disp["offsets"], pd, out=yp, ws=ws[moe.OP_FFN])
        mark(4)
        moe.combine(p, yp, w, disp["slot_to_row"], out=y)
        mark(5)

    layer_ws = None if wr is not None else moe.workspace(p, moe.OP_LAYER, dev)

    def layer_step():
        if layer_ws is None:
            step()
        else:
            moe.layer(p, inp["x"], inp["logits"], pgu, pd, out=y, ws=layer_ws)

    warm_up(step, 2, 0.0)  # the stage pass's calls
    warm_steps = warm_up(layer_step, args.warmup, args.warmup_seconds)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = (t1 - t0) / args.steps
    # stage pass: the same steps with an event between stages
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = {s: sum(events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)) / args.steps
                for j, s in enumerate(stages)}

    cold = None
    if args.flush_mib > 0:
        # cold-cache pass: a scratch write larger than the 256 MiB last-level cache before
        # every step, the step timed by events recorded after the write and after the step
        # (the warm figure timed the same way is the stage pass's first-to-last event)
        scratch = torch.empty(args.flush_mib << 18, dtype=torch.int32, device=dev)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.fill_(1)
            step(cev[i])
        torch.cuda.synchronize()
        del scratch
        cold_ms = sum(cev[i][0].elapsed_time(cev[i][5]) for i in range(args.steps)) / args.steps
        warm_ms = sum(events[i][0].elapsed_time(events[i][5]) for i in range(args.steps)) / args.steps
        cold = {"ms_per_step": round(cold_ms, 4), "tokens_per_s": round(wl.T / cold_ms * 1e3, 1),
                "warm_ms_per_step_same_timing": round(warm_ms, 4),
                "stages_us": {s: round(sum(cev[i][j].elapsed_time(cev[i][j + 1])
                                           for i in range(args.steps)) / args.steps * 1e3, 2)
                              for j, s in enumerate(stages)},
                "flush_bytes": args.flush_mib << 20,
                "how": "each step after a scratch write of flush_bytes, timed by events between "
                       "the stages (as the stage pass)"}

    # the dispatch with the row copy (moe_dispatch with xp: the layout, then the token rows
    # gathered into expert order), timed on its own: the layer step folds the gather into
    # the gate/up GEMM's activation loads instead
    xp = torch.empty(tk, wl.H, dtype=dt, device=dev)
    drows = dict(disp, xp=xp)
    keep_in = routing[2] if wl.capacity > 0 else None
    for _ in range(3):
        moe.dispatch(p, inp["x"], routing[0], keep_in, out=drows, ws=ws[moe.OP_DISPATCH], rows=True)
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        dev_[i][0].record()
        moe.dispatch(p, inp["x"], routing[0], keep_in, out=drows, ws=ws[moe.OP_DISPATCH], rows=True)
        dev_[i][1].record()
    torch.cuda.synchronize()
    drows_ms = sum(e[0].elapsed_time(e[1]) for e in dev_) / args.steps
    del xp, drows

    N = int(disp["offsets"][-1].item())
    E_hit = int((disp["counts"] > 0).sum().item())
    alg = algorithmic(wl, N, E_hit, router=args.router)
    b_act = 4 if wl.dtype == "f32" else 2
    row_bytes = wl.T * wl.H * b_act + N * wl.H * b_act  # x rows in, their k copies out
    copy_ms = max(drows_ms - stage_ms["dispatch"], 1e-6)
    dispatch_rows = {
        "us": round(drows_ms * 1e3, 2), "bound": "hbm",
        "achieved": round((alg["dispatch"]["bytes"] + row_bytes) / (drows_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "frac": round((alg["dispatch"]["bytes"] + row_bytes) / (drows_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "row_copy_us": round(copy_ms * 1e3, 2),
        "row_copy_frac": round(row_bytes / (copy_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "how": "moe_dispatch with xp timed alone; the row copy is that time less the layout-only "
               "dispatch stage",
    }
    dom = max(("gate_up", "down", "dispatch", "combine", "route"), key=lambda s: stage_ms[s])
    roof = roofline_of(dom, alg, stage_ms[dom] / 1e3, wl.dtype)
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(wl.name, dom)
    per_stage = {s: dict(us=round(stage_ms[s] * 1e3, 2),
                         **{k: v for k, v in roofline_of(s, alg, stage_ms[s] / 1e3, wl.dtype).items()
                            if k in ("bound", "achieved", "unit", "frac")}) for s in stages}
    backward = None
    if args.backward:
        backward = time_backward(args, moe, p, wl, inp, pgu, pd, routing, disp, yp, dev)
    layer_calls = None
    if args.chunk_tokens > 0:
        layer_calls = time_layer_calls(args, moe, p, wl, inp, pgu, pd, dev)
    out = {
        "metric": METRIC, "value": round(wl.T / sec, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm_steps,
        "ms_per_step": round(sec * 1e3, 4),
        "step_call": "moe_layer" if layer_ws is not None else "staged (moe_router first)",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded; routing logits and weights drawn per the workload recipe)",
        "config": {"workload": wl.name + ("+router" if args.router else ""), "T": wl.T, "H": wl.H, "E": wl.E, "k": wl.k, "I": wl.I,
                   "capacity": wl.capacity, "N_kept": N, "experts_hit": E_hit},
        "roofline": roof, "stages": per_stage,
    }
    out["dispatch_rows"] = dispatch_rows
    if cold is not None:
        out["cold_cache"] = cold
    if layer_calls is not None:
        out["layer_calls"] = layer_calls
    if backward is not None:
        out["backward"] = backward
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds, wr, groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
