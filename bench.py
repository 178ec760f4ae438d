"""Benchmark of the MoE expert-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_bf16]

A step is one whole forward (route -> permute -> fc1 + SwiGLU -> fc2 -> unpermute) over one batch
of seeded synthetic inputs already resident in HBM.  Before every timed step a 1 GiB buffer is
overwritten so that neither the L2s nor the 256 MiB Infinity Cache hold operands of the previous
step (the profiling rule of the page "MC2 通算融合架构总览", §8: flush L2 before every timed round).
Each step is bracketed by HIP events on the stream the library launches on; the flush is outside
the brackets.  A second pass of the same steps records every kernel of the library between events
(moe_timing_*), which gives each kernel's average duration for the roofline figures.

The flush reads the 1 GiB buffer by default (`--flush write` overwrites it instead): either way no
operand of the previous step stays in the L2s or the Infinity Cache, but a write flush also leaves
those caches full of dirty lines, whose write-back then lands on whichever kernel runs first.

Beside the step, and outside its figures: the router in front of the layer and, for the bfloat16
workloads, the layer's backward (gradients of x, the three weight stacks and probs, with g and u
recomputed), each timed on its own with the same flush; the permute and unpermute kernels on their
own, launched back to back from a captured HIP graph over rotating copies of their operands that
together outgrow the Infinity Cache (so neither the host's launch gap nor a warm cache enters their
rates); and, when the headline is the Mixtral layer, compact runs of the other three workloads (one
EP rank's grouped FFN, the fine-grained layer, the MX-FP8 layer) under the key "workloads".

Prints one JSON line on stdout; progress goes to stderr.
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

PEAK = {"bf16": 2500.0, "mxfp8": 5000.0, "f32": 157.3}     # dense TFLOP/s, MI355X published
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "moe_expert_layer_amd", "csrc")
METRIC = "MoE layer fwd tokens/s + grouped-GEMM % MFMA peak, Mixtral-shaped E=8 top-2"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_flops(M, H, F):
    """Algorithmic FLOPs of the routed rows: fc1 gate + up (2 * 2MHF) and fc2 (2MHF)."""
    return {"fc1": 4.0 * M * H * F, "fc2": 2.0 * M * H * F}


def byte_model(inp, M):
    """Algorithmic HBM bytes of the data-movement kernels (each row moved once per use)."""
    T, H, k = inp.T, inp.H, inp.k
    if inp.dtype == "mxfp8":
        row = H + H // 32
        return {"permute": (1 + k) * T * H + 4 * M, "permute_scale": (1 + k) * T * (H // 32),
                "unpermute": k * T * H * 2 + T * H * 2 + 8 * M}
    b = 4 if inp.dtype == "f32" else 2
    return {"permute": (1 + k) * T * H * b + 4 * M, "unpermute": (k * T * H * b + T * H * b + 8 * M)}


def _strip_probe(text: str) -> str:
    """The source as the product library compiles it: without the probe build's code (the
    `#ifdef MOE_PHASE_PROBE` blocks and their directives, keeping an `#else` part, the
    `MOE_PROBE(...)` uses and the macro's own definition)."""
    out, stack = [], []                 # per open #if: [probe block, in its #else part]
    live = lambda: all(not p or e for p, e in stack)
    for line in text.splitlines():
        d = line.strip()
        if d.startswith("#if"):
            stack.append([d.split()[:2] == ["#ifdef", "MOE_PHASE_PROBE"], False])
            if not stack[-1][0] and live():
                out.append(line)
        elif d.startswith("#else") and stack:
            stack[-1][1] = True
            if not stack[-1][0] and live():
                out.append(line)
        elif d.startswith("#endif") and stack:
            probe = stack.pop()[0]
            if not probe and live():
                out.append(line)
        elif live() and not d.startswith("#define MOE_PROBE"):
            out.append(line)
    text = "\n".join(out)
    while True:                                   # MOE_PROBE( ... ) with nested parentheses
        i = text.find("MOE_PROBE(")
        if i < 0:
            return text
        j, n = i + len("MOE_PROBE("), 1
        while n:
            n += {"(": 1, ")": -1}.get(text[j], 0)
            j += 1
        text = text[:i] + text[j:]


def _code_only(text: str) -> str:
    """C++ source without its comments, blank lines and probe-build code (a comment edit, or a
    change to the probe build, does not change a product kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = "\n".join(re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    text = _strip_probe(text)
    return "\n".join(line for line in text.splitlines() if line.strip())


def kernel_source_digest(files) -> str:
    """sha256 over the code (comments and blank lines dropped) of the named kernel sources, the
    shared headers and the tile-table builder (task order changes the traffic), to tie counter
    figures to code."""
    import hashlib
    h = hashlib.sha256()
    for f in list(files) + ["common.h", "internal.h", "gemm_common.h", "route.hip"]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _profile_summary(workload: str, kernel: str, what: str):
    """key = value pairs of the committed counter summary profiles/<kernel>_<workload>_<what>.txt,
    or None when there is none or the kernel sources changed since its counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_{what}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.split("#", 1)[0].strip()
    try:
        if kv.get("source_digest") != kernel_source_digest(kv["sources"].split(",")):
            return None
    except (KeyError, OSError):
        return None
    return kv


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when there is
    none for this workload or the kernel sources changed since the counters were taken."""
    kv = _profile_summary(workload, kernel, "traffic")
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def measured_clock(workload: str, kernel: str, achieved: float, peak: float):
    """The shader clock and matrix-core busy fraction that a counter run of the same kernel saw,
    and the live figure against the peak scaled to that clock (the chip is power-limited below the
    2.4 GHz the published peaks assume).  Empty when no current summary exists."""
    kv = _profile_summary(workload, kernel, "clock")
    try:
        sclk = float(kv["sclk_mhz_median"])
        return {"sclk_mhz": sclk, "peak_at_sclk": peak * sclk / 2400.0,
                "frac_at_sclk": achieved / (peak * sclk / 2400.0),
                "mfma_busy": float(kv["mfma_busy_median"])}
    except (TypeError, KeyError, ValueError):
        return {}


def cpu_baseline(inp, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload's tokens: the sample
    doubles until one run takes at least half the budget (or covers every token)."""
    import oracle
    rng = np.random.default_rng(123)
    order = rng.permutation(inp.T).astype(np.int32)
    n = 8
    while True:
        t0 = time.perf_counter()
        oracle.forward_tokens(inp, order[:n])
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or n >= inp.T:
            break
        n = min(inp.T, max(2 * n, int(n * budget_s / 2 / max(dt, 1e-3))))
    # the expert arithmetic those tokens carry: gate, up and down, 2 H F each, for each of k slots
    gflops = n * inp.k * 6.0 * inp.H * inp.F / dt / 1e9
    return {"value": n / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "gflops": gflops,
            "sample": f"{n} of {inp.T} tokens through the per-token definition (all k experts of each, "
                      f"weights decoded per call), {dt:.1f} s, fp64; gflops counts 6 H F per slot"}


def cpu_baseline_grouped(g, budget_s: float):
    """The oracle on a bounded sample of one EP rank's received rows (doubling as above)."""
    import oracle
    M = int(g.group_offsets[-1])
    rng = np.random.default_rng(123)
    order = rng.permutation(M)
    n = 8
    while True:
        t0 = time.perf_counter()
        oracle.grouped_ffn(g, row_index=np.sort(order[:n]))
        dt = time.perf_counter() - t0
        if dt >= budget_s / 2 or n >= M:
            break
        n = min(M, max(2 * n, int(n * budget_s / 2 / max(dt, 1e-3))))
    gflops = n * 6.0 * g.H * g.F / dt / 1e9                  # gate, up and down per row
    return {"value": n / dt, "unit": "rows/s", "cores": oracle.num_threads(), "kind": "oracle",
            "gflops": gflops,
            "sample": f"{n} of {M} received rows through their experts (weights decoded per call), "
                      f"{dt:.1f} s, fp64; gflops counts 6 H F per row"}


def graph_rate(torch, launches, sets, flush, repeats=3):
    """Mean duration of one launch when `launches` (callables, one per buffer set) run back to back
    from a captured HIP graph, several rounds over the sets: no host launch gap between kernels, and
    since the sets together outgrow the 256 MiB Infinity Cache, no launch finds its operands cached.
    The cache flush runs before each replay, outside the events."""
    for fn in launches:
        fn()
    torch.cuda.synchronize()
    rounds = max(2, -(-16 // len(launches)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        for _ in range(rounds):
            for fn in launches:
                fn()
    torch.cuda.synchronize()
    n = rounds * len(launches)
    times = []
    for _ in range(repeats):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / n)
    del g
    return float(np.median(times)), n, sets


def movement_rates(torch, mel, inp, d, dev, flush, bytes_):
    """permute (the standalone kernel; the forward folds it into fc1 where it can) and unpermute on
    their own, timed by graph_rate over rotating copies of their operands."""
    T, H, k, E = inp.T, inp.H, inp.k, inp.E
    M = T * k
    _, _, _, pos, _ = mel.route(d.expert_ids, E)
    mx = inp.dtype == "mxfp8"
    ydt = torch.float32 if inp.dtype == "f32" else torch.bfloat16
    out = {}
    # permute: x (and scales) in, x_perm (and scales) out
    set_bytes = bytes_["permute"] + bytes_.get("permute_scale", 0)
    S = max(2, -(-(768 << 20) // set_bytes))
    xs = [d.x.clone() for _ in range(S)]
    xss = [d.x_scale.clone() for _ in range(S)] if mx else [None] * S
    xp = [torch.empty((M, H), dtype=d.x.dtype, device=dev) for _ in range(S)]
    xps = [torch.empty((M, H // 32), dtype=torch.uint8, device=dev) for _ in range(S)] if mx else [None] * S
    launches = [lambda i=i: mel.permute(xs[i], pos, k, E=E, x_scale=xss[i], x_perm=xp[i],
                                        x_perm_scale=xps[i]) for i in range(S)]
    ms, n, _ = graph_rate(torch, launches, S, flush)
    ref = mel.permute(xs[0], pos, k, E=E, x_scale=xss[0])
    ok = torch.equal(ref[0] if mx else ref, xp[0])
    out["permute"] = {"us": ms * 1e3, "bytes": set_bytes, "GB/s": set_bytes / (ms * 1e-3) / 1e9,
                      "frac": set_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "launches": n,
                      "buffer_sets": S, "graph_equals_eager": bool(ok)}
    del xs, xss, xp, xps
    # unpermute: y_perm in, out out
    ub = bytes_["unpermute"]
    S = max(2, -(-(768 << 20) // ub))
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    ys = [torch.randn((M, H), generator=gen, device=dev).to(ydt) for _ in range(S)]
    os_ = [torch.empty((T, H), dtype=ydt, device=dev) for _ in range(S)]
    launches = [lambda i=i: mel.unpermute(ys[i], pos, d.probs, E=E, out=os_[i]) for i in range(S)]
    ms, n, _ = graph_rate(torch, launches, S, flush)
    ok = torch.equal(mel.unpermute(ys[0], pos, d.probs, E=E), os_[0])
    out["unpermute"] = {"us": ms * 1e3, "bytes": ub, "GB/s": ub / (ms * 1e-3) / 1e9,
                        "frac": ub / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "launches": n,
                        "buffer_sets": S, "graph_equals_eager": bool(ok)}
    del ys, os_
    # the ceiling at these sizes: a plain device copy moving the same number of bytes (half read,
    # half written), timed the same way over its own rotating buffers
    for name in ("permute", "unpermute"):
        nbytes = out[name]["bytes"]
        half = (nbytes // 2 + 15) // 16 * 16
        S = max(2, -(-(768 << 20) // nbytes))
        srcs = [torch.empty(half, dtype=torch.uint8, device=dev).fill_(1) for _ in range(S)]
        dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(S)]
        launches = [lambda i=i: dsts[i].copy_(srcs[i]) for i in range(S)]
        ms, _, _ = graph_rate(torch, launches, S, flush)
        cgbs = 2 * half / (ms * 1e-3) / 1e9
        out[name]["copy_same_bytes_GB/s"] = cgbs
        out[name]["copy_same_bytes_frac"] = cgbs / HBM_PEAK_GBS
        out[name]["frac_of_copy"] = out[name]["GB/s"] / cgbs
        del srcs, dsts
    torch.cuda.synchronize()
    log("standalone: " + ", ".join(f"{k_} {v['us']:.1f} us {v['GB/s']:.0f} GB/s ({100 * v['frac']:.0f}%; "
                                   f"a copy of the same bytes {v['copy_same_bytes_GB/s']:.0f} GB/s)"
                                   for k_, v in out.items()))
    return out


def bench_grouped(args, torch, mel, synth, dv, dev, name=None, compact=False):
    """One EP rank's share: the grouped FFN over rows as the dispatch All-to-All delivers them
    (source-major groups of 2 local experts); a step is one moe_grouped_ffn call, the metric rows/s.
    Returns the result dict (compact: no oracle baseline)."""
    name = name or args.workload
    g = synth.make_workload(name)
    M, H = g.rows.shape
    F, G = g.F, g.group_expert.shape[0]
    head = args.head_m_size if args.head_m_size is not None else 0
    rows = dv.tensor(g.rows, dev)
    offs, gexp = dv.tensor(g.group_offsets, dev), dv.tensor(g.group_expert, dev)
    wg, wu, wd = (dv.tensor(w, dev) for w in (g.w_gate, g.w_up, g.w_down))
    ws = torch.empty(max(mel.grouped_ffn_workspace_size(mel.problem(0, H, F, g.E_local, 1, mel.BF16, h), M, G)
                         for h in (head, 512)), dtype=torch.uint8, device=dev)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev).view(torch.float32)
    if args.copy_calibration_mib and not compact:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src

    def step(h):
        mel.grouped_ffn(rows, offs, gexp, wg, wu, wd, head_m_size=h, workspace=ws, out=out)

    for _ in range(args.warmup):
        step(head)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        if not args.no_flush:
            flush.sum()
        a.record()
        step(head)
        b.record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    mel.timing_reset()
    mel.timing_enable(True)
    for _ in range(args.steps):
        if not args.no_flush:
            flush.sum()
        step(head)
    kern = mel.timing_collect()
    mel.timing_enable(False)
    kavg = {n: tot / cnt for n, (tot, cnt) in kern.items()}
    ms_per_step = float(ms.mean())
    log(f"ms/step mean {ms_per_step:.3f} median {np.median(ms):.3f}; kernel avg ms: " +
        ", ".join(f"{n}={v:.4f}" for n, v in sorted(kavg.items())))
    fl = gemm_flops(M, H, F)
    fc1_ms, fc2_ms = kavg["fc1_bf16"], kavg["fc2_bf16"]
    peak = PEAK["bf16"]
    achieved = fl["fc1"] / (fc1_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC, "value": M / (ms_per_step * 1e-3), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "rows": M, "H": H, "F": F, "local_experts": g.E_local,
                   "sources": g.sources, "groups": G, "head_m_size": head,
                   "flush": "none" if args.no_flush else "read"},
        "gemm": {"tflops": (fl["fc1"] + fl["fc2"]) / ((fc1_ms + fc2_ms) * 1e-3) / 1e12,
                 "frac_of_peak": (fl["fc1"] + fl["fc2"]) / ((fc1_ms + fc2_ms) * 1e-3) / 1e12 / peak,
                 "peak_tflops": peak, "fc1_ms": fc1_ms, "fc2_ms": fc2_ms},
        "kernels_ms": kavg,
        "roofline": {"kernel": "fc1_bf16", "bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(name, "fc1_bf16"),
                     "per_launch": f"{fl['fc1']:.4g} FLOP = 4*M*H*F, M={M} received rows",
                     **measured_clock(name, "fc1_bf16", achieved, peak)},
        "timing": {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
                   "p90_ms": float(np.percentile(ms, 90))},
    }
    if not args.skip_chunked:
        for _ in range(2):
            step(512)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for a, b in cev:
            if not args.no_flush:
                flush.sum()
            a.record()
            step(512)
            b.record()
        torch.cuda.synchronize()
        cms = float(np.mean([a.elapsed_time(b) for a, b in cev]))
        result["chunked"] = {"head_m_size": 512, "ms_per_step": cms, "rows_per_s": M / (cms * 1e-3),
                             "overhead_vs_unchunked": cms / ms_per_step - 1.0}
        log(f"chunked(512) ms/step {cms:.3f}")
    if not args.skip_cpu_baseline and not compact:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        result["cpu_baseline"] = cpu_baseline_grouped(g, args.cpu_seconds)
    del rows, offs, gexp, wg, wu, wd, ws, out, flush
    torch.cuda.empty_cache()
    return result


def expert_roofline_ms(inp, counts, peak_tflops):
    """Attainable GEMM time by a per-expert roofline: each expert is bound by its FLOPs at the MFMA
    peak or by its bytes (its three weight matrices once, its rows into and out of both
    projections) at the HBM peak, whichever is larger; summed over the experts."""
    H, F = inp.H, inp.F
    eb = 1 if inp.dtype == "mxfp8" else 2
    t = 0.0
    for m in counts:
        m = float(m)
        if m == 0:
            continue
        flops = 6.0 * m * H * F
        byts = 3.0 * H * F * eb + m * (H * eb + 2 * F * eb + H * 2)
        t += max(flops / (peak_tflops * 1e12), byts / (HBM_PEAK_GBS * 1e9))
    return t * 1e3


def compact_layer(args, torch, mel, synth, dv, dev, name, flush):
    """A layer workload beside the headline: mean step time unchunked and chunked by 512 rows, the
    GEMMs' rate from per-kernel events, and the standalone permute / unpermute rates."""
    log(f"[{name}] generating inputs")
    inp = synth.make_workload(name)
    d = dv.layer(inp)
    T, H, F, E, k = inp.T, inp.H, inp.F, inp.E, inp.k
    M = T * k
    code = {"f32": mel.F32, "bf16": mel.BF16, "mxfp8": mel.MXFP8}[inp.dtype]
    ws = torch.empty(max(mel.workspace_size(mel.problem(T, H, F, E, k, code, h)) for h in (0, 512)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def step(h):
        if inp.dtype == "mxfp8":
            mel.expert_forward_mx(d.x, d.x_scale, d.w_gate, d.wg_scale, d.w_up, d.wu_scale,
                                  d.w_down, d.wd_scale, d.expert_ids, d.probs, head_m_size=h,
                                  out=out, workspace=ws)
        else:
            mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs,
                               head_m_size=h, out=out, workspace=ws)

    steps = min(args.steps, 10)
    for _ in range(3):
        step(0)
    modes = {}
    for h in (0, 512):
        step(h)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            flush()
            a.record()
            step(h)
            b.record()
        torch.cuda.synchronize()
        modes[h] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    mel.timing_reset()
    mel.timing_enable(True)
    for _ in range(steps):
        flush()
        step(0)
    kern = mel.timing_collect()
    mel.timing_enable(False)
    kavg = {n: tot / cnt for n, (tot, cnt) in kern.items()}
    suffix = {"bf16": "bf16", "mxfp8": "mx"}[inp.dtype]
    fl = gemm_flops(M, H, F)
    fc1_ms, fc2_ms = kavg[f"fc1_{suffix}"], kavg[f"fc2_{suffix}"]
    peak = PEAK[inp.dtype]
    tflops = (fl["fc1"] + fl["fc2"]) / ((fc1_ms + fc2_ms) * 1e-3) / 1e12
    counts = np.bincount(inp.expert_ids.ravel(), minlength=E)
    bound_ms = expert_roofline_ms(inp, counts, peak)
    bytes_ = byte_model(inp, M)
    from_bf16 = None
    if inp.dtype == "mxfp8":
        # the same layer fed the bfloat16 x, encoded by the library on its way into the gather
        xb = dv.tensor(inp.x_bf16, dev)
        wsq = torch.empty(mel.workspace_size(mel.problem(T, H, F, E, k, code, 0, mel.FLAG_QUANTIZE_X)),
                          dtype=torch.uint8, device=dev)

        def qstep():
            mel.expert_forward_mx(xb, None, d.w_gate, d.wg_scale, d.w_up, d.wu_scale, d.w_down,
                                  d.wd_scale, d.expert_ids, d.probs, out=out, workspace=wsq)

        qstep()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            flush()
            a.record()
            qstep()
            b.record()
        torch.cuda.synchronize()
        qms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        mel.timing_reset()
        mel.timing_enable(True)
        for _ in range(steps):
            flush()
            qstep()
        qk = mel.timing_collect()
        mel.timing_enable(False)
        enc_ms = qk["mx_encode_x"][0] / qk["mx_encode_x"][1]
        enc_bytes = T * H * 2 + T * H + T * (H // 32)
        from_bf16 = {"ms_per_step": qms, "tokens_per_s": T / (qms * 1e-3),
                     "mx_encode_x_us": enc_ms * 1e3,
                     "mx_encode_x_GB/s": enc_bytes / (enc_ms * 1e-3) / 1e9}
        log(f"[{name}] from bf16 x: ms/step {qms:.3f}, encode {enc_ms * 1e3:.1f} us")
        del xb, wsq
    res = {
        "config": {"T": T, "H": H, "F": F, "E": E, "k": k, "dtype": inp.dtype, "routed_rows": M},
        "ms_per_step": modes[0], "tokens_per_s": T / (modes[0] * 1e-3),
        "chunked_512": {"ms_per_step": modes[512], "tokens_per_s": T / (modes[512] * 1e-3)},
        "gemm": {"tflops": tflops, "frac_of_peak": tflops / peak, "peak_tflops": peak,
                 "fc1_ms": fc1_ms, "fc2_ms": fc2_ms,
                 "expert_roofline_ms": bound_ms,
                 "frac_of_expert_roofline": bound_ms / (fc1_ms + fc2_ms)},
        "kernels_ms": kavg,
        "hbm_in_step": {n: {"GB/s": bytes_[n] / (kavg[n] * 1e-3) / 1e9,
                            "frac": bytes_[n] / (kavg[n] * 1e-3) / 1e9 / HBM_PEAK_GBS}
                        for n in bytes_ if n in kavg},
        "hbm_standalone": movement_rates(torch, mel, inp, d, dev, flush, bytes_),
    }
    if from_bf16 is not None:
        res["from_bf16_x"] = from_bf16
    log(f"[{name}] ms/step {modes[0]:.3f} (chunked {modes[512]:.3f}); GEMMs {tflops:.0f} TFLOP/s "
        f"({100 * tflops / peak:.1f}% of peak, {100 * bound_ms / (fc1_ms + fc2_ms):.0f}% of the per-expert roofline)")
    del d, ws, out
    torch.cuda.empty_cache()
    return res


EXTRA_WORKLOADS = ("ep_rank_bf16", "finegrained_bf16", "mxfp8")


PROBE_FIELDS = ("wait", "loop", "loop_full", "sync", "setup", "epilogue", "tasks", "tasks_full",
                "total", "realtime", "workgroups", "steps")
PROBE_KINDS = ("fc2_bf16", "fc1_bf16", "recompute_gu", "wgrad", "dgrad_down", "dgrad_gate_up",
               "fc2_mx", "fc1_mx")


def phase_probe(args, torch, mel, synth, dv, dev):
    """Per-task phases of the large-tile GEMM launches, from the probe library's cycle stamps: the
    forward (or the EP rank's grouped FFN) run --steps times after --warmup, each call after the
    cache flush the timed benchmark uses; then, for bf16 layer workloads and unless --skip-backward,
    the backward (recomputing g and u) the same way.  Cycles are wave 0's counter cycles; a bf16 K
    step (32) issues 2 waves x 16 MFMAs x 32 cycles and an MX one (64) 2 waves x 8 MFMAs x 64
    cycles, 1024 cycles per SIMD either way, so loop_mfma_fraction is (K steps x 1024) / K-loop
    cycles, over the full-height tasks where tasks differ in height."""
    import ctypes
    lib = mel.library()
    probe = lib.moe_probe_phases
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int]
    probe.restype = ctypes.c_int
    cfg = synth.WORKLOADS[args.workload]
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev).view(torch.float32)
    head = args.head_m_size if args.head_m_size is not None else 0
    legs = []
    if cfg["kind"] == "grouped":
        g = synth.make_workload(args.workload)
        M, H = g.rows.shape
        rows = dv.tensor(g.rows, dev)
        offs, gexp = dv.tensor(g.group_offsets, dev), dv.tensor(g.group_expert, dev)
        wg, wu, wd = (dv.tensor(w, dev) for w in (g.w_gate, g.w_up, g.w_down))
        out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        legs.append(("forward", lambda: mel.grouped_ffn(rows, offs, gexp, wg, wu, wd, head_m_size=head, out=out)))
    else:
        inp = synth.make_workload(args.workload)
        if inp.dtype not in ("bf16", "mxfp8"):
            sys.exit("--phase-probe covers the bf16 and MX-FP8 GEMMs: pick such a workload")
        d = dv.layer(inp, dev)
        out = torch.empty((inp.T, inp.H), dtype=torch.bfloat16, device=dev)
        if inp.dtype == "mxfp8":
            legs.append(("forward", lambda: mel.expert_forward_mx(
                d.x, d.x_scale, d.w_gate, d.wg_scale, d.w_up, d.wu_scale, d.w_down, d.wd_scale,
                d.expert_ids, d.probs, head_m_size=head, out=out)))
        else:
            legs.append(("forward", lambda: mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids,
                                                               d.probs, head_m_size=head, out=out)))
        if not args.skip_backward and inp.dtype == "bf16":
            dout = dv.tensor(synth.make_dout(inp), dev)
            bws = torch.empty(mel.backward_workspace_size(mel.problem(inp.T, inp.H, inp.F, inp.E, inp.k, mel.BF16)),
                              dtype=torch.uint8, device=dev)
            legs.append(("backward", lambda: mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids,
                                                                 d.probs, dout, workspace=bws)))
    report = {"workload": args.workload, "steps": args.steps, "head_m_size": head, "kernels": {}}
    nf = len(PROBE_FIELDS)
    for leg, step in legs:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        if probe(None, 1) != 0:
            raise RuntimeError("moe_probe_phases failed")
        for _ in range(args.steps):
            if not args.no_flush:
                flush.sum()
            step()
        buf = (ctypes.c_ulonglong * (len(PROBE_KINDS) * nf))()
        if probe(ctypes.cast(buf, ctypes.c_void_p), 1) != 0:
            raise RuntimeError("moe_probe_phases failed")
        for kind, name in enumerate(PROBE_KINDS):
            v = dict(zip(PROBE_FIELDS, buf[kind * nf:(kind + 1) * nf]))
            if v["tasks"] == 0:
                continue
            steps_per_task = v["steps"] / v["tasks"]
            full = v["tasks_full"] > 0 and v["loop_full"] > 0
            r = {"leg": leg,
                 "tasks_per_launch": v["tasks"] / args.steps,
                 "tasks_per_workgroup": v["tasks"] / v["workgroups"],
                 "k_steps_per_task": steps_per_task,
                 "per_task_cycles": {f: v[f] / v["tasks"] for f in ("wait", "loop", "sync", "setup", "epilogue")},
                 "share_of_workgroup_cycles": {f: v[f] / v["total"] for f in ("wait", "loop", "sync", "setup", "epilogue")},
                 "loop_full_cycles": v["loop_full"] / v["tasks_full"] if full else None,
                 "mfma_issue_cycles_per_task": steps_per_task * 1024,
                 "loop_mfma_fraction": (steps_per_task * 1024 * v["tasks_full"] / v["loop_full"] if full
                                        else v["steps"] * 1024 / v["loop"]),
                 "counter_mhz": v["total"] / v["realtime"] * 100.0 if v["realtime"] else None,
                 "workgroup_us": v["realtime"] / v["workgroups"] / 100.0}
            report["kernels"][name] = r
            pt = r["per_task_cycles"]
            log(f"{name}: {r['tasks_per_workgroup']:.1f} tasks per workgroup, {steps_per_task:.0f} K steps; per task "
                f"wait {pt['wait']:.0f}, K loop {pt['loop']:.0f} (MFMA issue {r['loop_mfma_fraction']:.3f} of it"
                f"{' on full tasks' if full else ''}), sync {pt['sync']:.0f}, setup {pt['setup']:.0f}, "
                f"epilogue {pt['epilogue']:.0f} counter cycles; counter {r['counter_mhz'] or 0:.0f} MHz")
    return {"phase_probe": report}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--head-m-size", type=int, default=None,
                    help="chunk rows for the reported mode (default: unchunked)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--flush", choices=["read", "write"], default="read",
                    help="how the 1 GiB buffer evicts the caches between steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-chunked", action="store_true")
    ap.add_argument("--skip-router", action="store_true")
    ap.add_argument("--skip-backward", action="store_true")
    ap.add_argument("--separate-permute", action="store_true",
                    help="run the permute step as its own kernel instead of inside fc1's row loads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (reference for HBM counters)")
    ap.add_argument("--skip-workloads", action="store_true",
                    help="leave out the compact runs of the other workloads beside the Mixtral headline")
    ap.add_argument("--skip-standalone", action="store_true",
                    help="leave out the standalone permute / unpermute rates")
    ap.add_argument("--mx-from-bf16", action="store_true",
                    help="MX workloads: feed the bfloat16 x and let the library encode it (MOE_FLAG_QUANTIZE_X)")
    ap.add_argument("--phase-probe", action="store_true",
                    help="bf16 workloads: run the forward on the probe library (per-task cycle stamps in "
                         "the bf16 GEMMs) and print a per-task phase report instead of the benchmark line")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_expert_layer_amd as mel
    import synth
    from synth import device as dv

    if args.phase_probe:
        from moe_expert_layer_amd.build import PROBE_LIB_PATH
        if not os.path.exists(PROBE_LIB_PATH):
            sys.exit(f"{PROBE_LIB_PATH} is missing: build it with `python -m moe_expert_layer_amd.build`")
        mel.library(PROBE_LIB_PATH)        # loaded first, so every call below runs the probe build
    if not os.path.exists(mel.lib_path):
        from moe_expert_layer_amd.build import build
        build()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    cfg = synth.WORKLOADS[args.workload]
    if args.phase_probe:
        print(json.dumps(phase_probe(args, torch, mel, synth, dv, dev)), flush=True)
        return
    if cfg["kind"] == "grouped":
        print(json.dumps(bench_grouped(args, torch, mel, synth, dv, dev)), flush=True)
        return
    log(f"generating {args.workload} inputs")
    t0 = time.perf_counter()
    inp = synth.make_workload(args.workload)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    d = dv.layer(inp, dev)
    T, H, F, E, k = inp.T, inp.H, inp.F, inp.E, inp.k
    M = T * k
    head = args.head_m_size if args.head_m_size is not None else 0
    code = {"f32": mel.F32, "bf16": mel.BF16, "mxfp8": mel.MXFP8}[inp.dtype]
    qflag = mel.FLAG_QUANTIZE_X if (inp.dtype == "mxfp8" and args.mx_from_bf16) else 0
    ws_bytes = max(mel.workspace_size(mel.problem(T, H, F, E, k, code, h, qflag)) for h in (head, 512))
    xb16 = dv.tensor(inp.x_bf16, dev) if qflag else None
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32 if inp.dtype == "f32" else torch.bfloat16,
                      device=dev)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    flush_words = flush.view(torch.float32)     # summed as float: no widening copy of the buffer

    def do_flush():
        if args.no_flush:
            return
        if args.flush == "write":
            flush.fill_(1)
        else:
            flush_words.sum()

    def step(h):
        if inp.dtype == "mxfp8":
            mel.expert_forward_mx(xb16 if qflag else d.x, None if qflag else d.x_scale, d.w_gate,
                                  d.wg_scale, d.w_up, d.wu_scale, d.w_down, d.wd_scale,
                                  d.expert_ids, d.probs, head_m_size=h, out=out, workspace=ws,
                                  separate_permute=args.separate_permute)
        else:
            mel.expert_forward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs,
                               head_m_size=h, out=out, workspace=ws,
                               separate_permute=args.separate_permute)

    def timed(h, steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for a, b in ev:
            do_flush()
            a.record()
            step(h)
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return np.array([a.elapsed_time(b) for a, b in ev]), wall

    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(head)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps (head_m_size={head})")
    ms, wall = timed(head, args.steps)
    ms_per_step = float(ms.mean())
    log(f"ms/step mean {ms_per_step:.3f} median {np.median(ms):.3f} p10 {np.percentile(ms, 10):.3f} "
        f"p90 {np.percentile(ms, 90):.3f}")

    # per-kernel durations, same steps, events around every kernel the library launches
    mel.timing_reset()
    mel.timing_enable(True)
    for _ in range(args.steps):
        do_flush()
        step(head)
    kern = mel.timing_collect()
    mel.timing_enable(False)
    kavg = {n: tot / cnt for n, (tot, cnt) in kern.items()}
    log("kernel avg ms: " + ", ".join(f"{n}={v:.4f}" for n, v in sorted(kavg.items())))

    fl = gemm_flops(M, H, F)
    suffix = {"f32": "f32", "bf16": "bf16", "mxfp8": "mx"}[inp.dtype]
    fc1_ms, fc2_ms = kavg.get(f"fc1_{suffix}", float("nan")), kavg.get(f"fc2_{suffix}", float("nan"))
    gemm_tflops = (fl["fc1"] + fl["fc2"]) / ((fc1_ms + fc2_ms) * 1e-3) / 1e12
    peak = PEAK[inp.dtype]
    bytes_ = byte_model(inp, M)
    dominant = max(kavg, key=kavg.get)
    dom_flops = fl.get(dominant.split("_")[0]) if dominant.startswith("fc") else None
    if dom_flops is not None:
        achieved = dom_flops / (kavg[dominant] * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s", "frac": achieved / peak,
                "traffic": measured_traffic(args.workload, dominant),
                "per_launch": f"{dom_flops:.4g} FLOP = 2*M*H*F per projection, M={M} routed rows",
                **measured_clock(args.workload, dominant, achieved, peak)}
    else:
        gbs = bytes_[dominant] / (kavg[dominant] * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "traffic": measured_traffic(args.workload, dominant)}
    hbm = {n: {"GB/s": bytes_[n] / (kavg[n] * 1e-3) / 1e9,
               "frac": bytes_[n] / (kavg[n] * 1e-3) / 1e9 / HBM_PEAK_GBS}
           for n in bytes_ if n in kavg}

    result = {
        "metric": METRIC, "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": inp.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "T": T, "H": H, "F": F, "E": E, "k": k,
                   "head_m_size": head, "routed_rows": M, "flush_bytes": 0 if args.no_flush else 1 << 30,
                   "flush": "none" if args.no_flush else args.flush,
                   "permute": "separate kernel" if args.separate_permute else "inside fc1 where the large tiles serve",
                   **({"x": "bfloat16, MX-encoded by the library"} if qflag else {})},
        "gemm": {"tflops": gemm_tflops, "frac_of_peak": gemm_tflops / peak, "peak_tflops": peak,
                 "fc1_ms": fc1_ms, "fc2_ms": fc2_ms},
        "kernels_ms": kavg, "hbm": hbm, "roofline": roof,
        "timing": {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
                   "p90_ms": float(np.percentile(ms, 90)),
                   "wall_ms_per_step_incl_flush": wall * 1e3 / args.steps},
    }

    # the router in front of the layer (top-k gate over this workload's logits), timed on its own:
    # the layer's step starts from expert ids, as the benchmark's metric does
    if not args.skip_router:
        kw = {key: cfg[key] for key in ("zipf_s", "n_zero") if key in cfg}
        logits = torch.from_numpy(
            synth.make_logits(T, E, cfg.get("routing", "normal_logits"), seed=0, **kw)).to(dev)
        for _ in range(3):
            mel.router_topk(logits, k)
        torch.cuda.synchronize()
        mel.timing_reset()
        mel.timing_enable(True)
        for _ in range(args.steps):
            do_flush()
            mel.router_topk(logits, k)
        rk = mel.timing_collect()
        mel.timing_enable(False)
        r_ms = rk["router"][0] / rk["router"][1]
        r_bytes = T * E * 4 + T * k * 8
        result["router"] = {"ms": r_ms, "bytes": r_bytes, "GB/s": r_bytes / (r_ms * 1e-3) / 1e9,
                            "frac": r_bytes / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"router {r_ms * 1e3:.1f} us ({r_bytes / (r_ms * 1e-3) / 1e9:.0f} GB/s)")

    # the layer's backward (bf16 workloads): gradients of sum(dout * out) for x, the three weight
    # stacks and probs, g and u recomputed inside; timed on its own like the router
    if not args.skip_backward and inp.dtype == "bf16":
        dout = dv.tensor(synth.make_dout(inp), dev)
        bws = torch.empty(mel.backward_workspace_size(mel.problem(T, H, F, E, k, mel.BF16)),
                          dtype=torch.uint8, device=dev)

        def bstep():
            return mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout,
                                       workspace=bws)

        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        bsteps = max(3, args.steps // 2)
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(bsteps)]
        for a, b in bev:
            do_flush()
            a.record()
            bstep()
            b.record()
        torch.cuda.synchronize()
        bms = np.array([a.elapsed_time(b) for a, b in bev])
        mel.timing_reset()
        mel.timing_enable(True)
        for _ in range(bsteps):
            do_flush()
            bstep()
        bk = mel.timing_collect()
        mel.timing_enable(False)
        bkavg = {n: tot / cnt for n, (tot, cnt) in bk.items()}
        grad_flops = 12.0 * M * H * F            # dgrad down + gate/up, wgrad down + gate/up
        rec_flops = 4.0 * M * H * F              # g and u recomputed
        gemm_names = ("recompute_gu", "dgrad_down", "dgrad_gate_up", "wgrad_down",
                      "wgrad_gate", "wgrad_up")
        gemm_ms = sum(bkavg.get(n, 0.0) for n in gemm_names)
        b_mean = float(bms.mean())
        result["backward"] = {
            "ms": b_mean, "median_ms": float(np.median(bms)), "steps": bsteps,
            "tokens_per_s": T / (b_mean * 1e-3),
            "gemm_tflops": (grad_flops + rec_flops) / (gemm_ms * 1e-3) / 1e12,
            "gemm_frac_of_peak": (grad_flops + rec_flops) / (gemm_ms * 1e-3) / 1e12 / peak,
            "flops": {"gradients": grad_flops, "recompute": rec_flops},
            "kernels_ms": bkavg,
        }
        log(f"backward ms/step {b_mean:.3f}; kernel avg ms: " +
            ", ".join(f"{n}={v:.4f}" for n, v in sorted(bkavg.items())))
        # training pair: the forward that keeps g and u, and the backward that takes them
        saved = torch.empty((2, M, F), dtype=torch.bfloat16, device=dev)

        def fstep():
            mel.expert_forward_train(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, out=out,
                                     saved_gu=saved, workspace=ws)

        def bstep_saved():
            return mel.expert_backward(d.x, d.w_gate, d.w_up, d.w_down, d.expert_ids, d.probs, dout,
                                       workspace=bws, saved_gu=saved)

        pair = {}
        for name, fn in (("forward_train_ms", fstep), ("backward_saved_gu_ms", bstep_saved)):
            fn()
            torch.cuda.synchronize()
            pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(bsteps)]
            for a, b in pev:
                do_flush()
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            pair[name] = float(np.mean([a.elapsed_time(b) for a, b in pev]))
        pair["step_ms"] = pair["forward_train_ms"] + pair["backward_saved_gu_ms"]
        pair["tokens_per_s"] = T / (pair["step_ms"] * 1e-3)
        result["backward"]["training_pair"] = pair
        log(f"forward keeping g, u {pair['forward_train_ms']:.3f} ms + backward on them "
            f"{pair['backward_saved_gu_ms']:.3f} ms")
        del bws, dout, saved

    if not args.skip_chunked:
        for _ in range(2):
            step(512)
        cms, _ = timed(512, args.steps)
        result["chunked"] = {"head_m_size": 512, "ms_per_step": float(cms.mean()),
                             "tokens_per_s": T / (float(cms.mean()) * 1e-3),
                             "overhead_vs_unchunked": float(cms.mean()) / ms_per_step - 1.0}
        log(f"chunked(512) ms/step {cms.mean():.3f}")

    if not args.skip_standalone and inp.dtype != "f32":
        result["hbm_standalone"] = movement_rates(torch, mel, inp, d, dev, do_flush, bytes_)

    if not args.skip_cpu_baseline:
        log(f"cpu baseline (~{args.cpu_seconds:.0f} s of oracle work)")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        log(f"cpu baseline {result['cpu_baseline']['value']:.2f} tokens/s on "
            f"{result['cpu_baseline']['cores']} threads")

    # the other workloads, compactly, beside the headline (same flush, no oracle baseline)
    if args.workload == "mixtral_bf16" and not args.skip_workloads:
        del d, ws, out
        torch.cuda.empty_cache()
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            if synth.WORKLOADS[name]["kind"] == "grouped":
                log(f"[{name}] grouped FFN")
                r = bench_grouped(args, torch, mel, synth, dv, dev, name=name, compact=True)
                result["workloads"][name] = {k_: r[k_] for k_ in ("value", "unit", "ms_per_step",
                                                                  "config", "gemm", "chunked",
                                                                  "kernels_ms") if k_ in r}
            else:
                result["workloads"][name] = compact_layer(args, torch, mel, synth, dv, dev, name,
                                                          do_flush)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
