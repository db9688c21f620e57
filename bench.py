"""Benchmark of the MoE layer with zero-computation experts on one MI355X.

One step = one forward of the layer as configured (router GEMM, softmax +
bias top-K, histogram, scan, permute, grouped GEMM gate/up + SwiGLU, grouped
GEMM down, combine with the identity experts and the residual), always with
the workload's own selection bias, followed by one moe_zc_bias_update (PID
step toward uniform load) from that routing, on the same stream.  The PID
step starts every timed step from the configured bias and zero controller
state, so each step times the same layer and the same single bias update;
the update is timed as a stage of its own.  A separate, untimed closed loop
(bias carried over repeated batches) is reported beside it.

Inputs are seeded and synthetic, resident in HBM before the timed region.
bf16 expert weights are packed once at setup (moe_zc_pack_expert_weights, as
at model load) and the step calls moe_zc_forward_packed; --layout rowmajor
times moe_zc_forward on the row-major weights instead.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload prefill]

The headline is --workload (default prefill, bf16).  The same run then times
the other workloads (tiny, mid, decode, skew in their own dtypes, and the
prefill layer with the block-FP8 gate/up projection) and the training step
of the prefill and skewed layers (as --pass backward times it), and reports
each under "workloads" (skip with --no-extra-workloads).

--pass backward times a training step of the layer instead: the packed
forward saving its routing and the expert pre-activations (aux.act), then
moe_zc_backward (dx, the router gradient and the fp32 expert weight
gradients) from them, with the backward also timed alone; --recompute uses
the row-major forward without saved pre-activations, so the backward
recomputes them.

Prints one JSON line.  Per-stage times come from HIP events that the library
records on the launch stream at its stage boundaries.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + activated TFLOP/s (% of bf16 MFMA peak) on 1 MI355X"
PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5.0e15       # dense fp8 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # HBM3E, B/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["tiny", "mid", "decode", "prefill", "skew"])
    ap.add_argument("--layout", default="packed", choices=["packed", "rowmajor"],
                    help="expert weight layout of the bf16 forward")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp8"],
                    help="fp8: gate/up projection in block FP8 (moe_zc_forward_packed_fp8); "
                         "the down projection stays bf16")
    ap.add_argument("--fp8-down", action="store_true",
                    help="with --precision fp8: the down projection in block FP8 as well")
    ap.add_argument("--pass", dest="which", default="forward", choices=["forward", "backward"],
                    help="backward: time forward + moe_zc_backward (a training step)")
    ap.add_argument("--recompute", action="store_true",
                    help="--pass backward: row-major forward, pre-activations recomputed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip measuring the box's stream bandwidths and dense GEMM rate")
    ap.add_argument("--cpu-experts", type=int, default=96,
                    help="experts the CPU-baseline sample evaluates")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a device copy of known size (for scaling counters)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the untimed HIP-graph replay of the step")
    ap.add_argument("--no-power-probe", action="store_true",
                    help="skip sampling socket power and clocks (amd-smi) on the headline")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time only the --workload layer (skip the other workloads)")
    ap.add_argument("--closed-loop-steps", type=int, default=10,
                    help="batches of the untimed closed-loop PID report")
    return ap.parse_args()


COUNTERS_MD = os.path.join(ROOT, "profiles", "gemm_gate_up_prefill_counters.md")
# the sources the packed GEMM kernel is compiled from (its epilogue and
# helpers live in the headers)
GEMM_SRC = [os.path.join(ROOT, "mixture_experts_layer_bias_amd", "csrc", f)
            for f in ("gemm_packed.hip", "gemm_tile.hpp", "common.hpp", "kernels.hpp")]


def source_sha(paths):
    """sha256 (first 16 hex digits) of the files' bytes, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken on another kernel
    source (the summary records the source hash it was measured on)."""
    if not os.path.exists(COUNTERS_MD):
        return None
    vals = {}
    for line in open(COUNTERS_MD):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    try:
        if vals.get("kernel source sha256") != source_sha(GEMM_SRC):
            return None
        return float(vals["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """A plain device-to-device copy of 2 GiB, three times: each launch reads
    and writes exactly 2 GiB, which scales the FETCH_SIZE / WRITE_SIZE
    counters of rocprofv3."""
    import torch
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}))


def measured_peaks(dev):
    """What this machine reaches on plain streams and a dense GEMM, measured before
    the inputs exist: a 8 GiB fill (writes), a 4 GiB copy (reads + writes),
    row sums of an 8 GiB [65536, 32768] matrix (reads; a single full reduction
    streams slower on this machine), and an 8192^3 bf16 matrix product from the
    vendor BLAS.  The fractions of the spec peaks are what the roofline uses;
    these put them in context."""
    import torch

    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / n

    out = {}
    buf = torch.empty(2 << 30, dtype=torch.float32, device=dev)          # 8 GiB
    out["hbm_write_GBps"] = buf.numel() * 4 / timed(lambda: buf.fill_(1.0)) / 1e9
    rows = buf.view(65536, 32768)                                      # row sums: a read stream
    out["hbm_read_GBps"] = buf.numel() * 4 / timed(lambda: rows.sum(dim=1)) / 1e9
    del rows
    del buf
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)  # 4 GiB
    dst = torch.empty_like(src)
    out["hbm_copy_GBps"] = 2 * src.numel() * 4 / timed(lambda: dst.copy_(src)) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    out["bf16_gemm_TFLOPs"] = 2.0 * n ** 3 / timed(lambda: torch.matmul(a, b)) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {k: round(v, 1) for k, v in out.items()}


def power_probe(step, seconds=4.0):
    """Socket power and graphics clocks while the step runs back to back
    (untimed), sampled with amd-smi in a thread of its own; None where the
    tool is missing.  Under the MI355X power cap the clocks the expert GEMMs
    run at are set by the energy they spend, which is what this records."""
    import re
    import shutil
    import subprocess
    import threading

    import torch

    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    samples = []
    stop = threading.Event()

    def sampler():
        time.sleep(0.8)                       # past the first steps
        while not stop.is_set():
            try:
                txt = subprocess.run([tool, "metric", "-p", "-c"], capture_output=True,
                                     text=True, timeout=10).stdout
            except Exception:
                return
            pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)", txt)
            clocks, section = [], ""
            for line in txt.splitlines():
                st = line.strip()
                if st.endswith(":") and not st.startswith("CLK"):
                    section = st[:-1]
                m_ = re.match(r"CLK:\s*([0-9.]+)\s*MHz", st)
                if m_ and section.startswith("GFX_"):
                    clocks.append(float(m_.group(1)))
            if pw:
                samples.append((float(pw.group(1)), clocks))

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        step()
        torch.cuda.synchronize()
        n += 1
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    watts = [w_ for w_, _ in samples]
    clk = [c for _, cs in samples for c in cs]
    return {"socket_W": watts, "gfx_clock_MHz_mean": (sum(clk) / len(clk)) if clk else None,
            "gfx_clock_MHz_min": min(clk) if clk else None, "samples": len(samples),
            "steps_run": n, "source": "amd-smi metric -p -c while the step runs back to back"}


def algorithmic(w, S, touched, es, fp8=False, fp8_down=False):
    """Algorithmic bytes / FLOPs per launch of each stage (inputs read once,
    outputs written once).  bf16: the gate/up GEMM gathers its rows from x,
    so its input is x itself and the grouping stage moves only indices.
    fp8: the gate/up weights are one byte per value plus one scale byte per
    32, and x (bf16) is read once to be quantized; the FP8 copy of x that the
    GEMM gathers is internal traffic and not counted."""
    T, d, I, N, E, K = w.T, w.d, w.I, w.N, w.E, w.K
    gathered = es == 2 and T * d * es < 2**31
    w_gu = touched * 2 * I * d * ((1.0 + 1.0 / 32.0) if fp8 else es)
    return {
        "router_gemm": {"flop": 2.0 * T * d * E,
                        "bytes": T * d * es + E * d * 4 + T * E * 4},
        "softmax_topk": {"bytes": T * E * 4 + E * 4 + T * K * 8},
        "permute": {"bytes": T * K * 4 * 4 if gathered else
                    T * d * es + S * d * es + T * K * 4 * 3},
        "gemm_gate_up_swiglu": {"flop": 4.0 * d * I * S,
                                "bytes": w_gu + (T if gathered else S) * d * es + S * I * es},
        "gemm_down": {"flop": 2.0 * d * I * S,
                      # FP8: the FP8 copy of h is internal traffic; h (bf16) is
                      # read once to be quantized
                      "bytes": touched * d * I * ((1.0 + 1.0 / 32.0) if fp8_down else es)
                      + S * I * es + S * d * es},
        "combine": {"bytes": S * d * es + 3 * T * d * es + T * K * 12},
    }


def cpu_baseline(w, inp, n_experts, weights):
    """The fp64 oracle on the host cores: routing of every token, the SwiGLU
    experts 0..n_experts-1 (``weights``: their host copies) with all their
    rows (scaled to all touched experts), and the combine of every token."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cores = min(threads, len(os.sched_getaffinity(0)))
    x = inp["x"].cpu()
    wr = inp["w_router"].cpu()
    b = inp["bias"].cpu().numpy()
    res = inp["residual"].cpu() if inp["residual"] is not None else None
    n_exp = min(n_experts, w.N, len(weights))
    t0 = time.perf_counter()
    l64 = oracle.router_logits(x, wr)
    rt = oracle.route(l64.astype(np.float32), b, w.K, w.N)
    t1 = time.perf_counter()
    idx = rt["idx"]
    x64 = oracle.moe_zc._f64(x)
    rows = np.zeros((w.T, w.K, w.d))
    for e in range(n_exp):
        tt, kk = np.nonzero(idx == e)
        rows[tt, kk] = oracle.swiglu_ffn(x64[tt], *weights[e])
    t2 = time.perf_counter()
    oracle.combine(x64, idx, rt["gate"], rows, w.N, res)
    t3 = time.perf_counter()
    touched = int((rt["loads"][: w.N] > 0).sum())
    sampled_rows = int(rt["loads"][:n_exp].sum())
    t_ffn = (t2 - t1) * touched / max(1, n_exp)
    total = (t1 - t0) + t_ffn + (t3 - t2)
    return {"value": w.T / total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"fp64 oracle: routing of all {w.T} tokens ({t1 - t0:.2f} s); SwiGLU "
                       f"experts 0..{n_exp - 1} with all their {sampled_rows} rows "
                       f"({t2 - t1:.2f} s), scaled by {touched}/{n_exp} touched experts; "
                       f"combine of all tokens ({t3 - t2:.2f} s); estimated layer time "
                       f"{total:.1f} s"),
            "seconds_measured": round(t3 - t0, 2)}


def bench_backward(args, w, dev, steps=None, warmup=None):
    """Training step = forward (routing saved) + backward; also the backward
    alone.  Returns the JSON record (steps and warmup default to the command
    line's).  FLOPs of the backward's expert products: q (2 d I S), the rows
    of dx (4 d I S), dW_down, dW_gate, dW_up (6 d I S), and with --recompute
    a and u again (4 d I S); router: dx term and dW_router (4 T d E)."""
    import torch

    import mixture_experts_layer_bias_amd as m
    from workloads import make_inputs, make_upstream_grad

    if w.dtype != "bf16":
        print("bench.py: the backward takes a bf16 workload", file=sys.stderr)
        sys.exit(2)
    inp = make_inputs(w, device=dev, residual=False)
    dy = make_upstream_grad(w, dev)
    tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    saved = not args.recompute
    if saved:  # packed weights for the forward; the row-major copies are no longer read
        gu, dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        torch.cuda.synchronize()
        for k in ("w_gate", "w_up", "w_down"):
            inp[k] = None
        torch.cuda.empty_cache()
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, dev, keys=m.AUX_KEYS + (("act",) if saved else ()),
                      I=w.I)
    y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device=dev)
    ws_f = torch.empty(m.moe_zc_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K, torch.bfloat16),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(m.moe_zc_backward_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K),
                       dtype=torch.uint8, device=dev)
    grads = {"dx": torch.empty(w.T, w.d, dtype=torch.bfloat16, device=dev),
             "dw_router": torch.empty(w.E, w.d, dtype=torch.float32, device=dev),
             "dw_gate": torch.empty(w.N, w.I, w.d, dtype=torch.float32, device=dev),
             "dw_up": torch.empty(w.N, w.I, w.d, dtype=torch.float32, device=dev),
             "dw_down": torch.empty(w.N, w.d, w.I, dtype=torch.float32, device=dev)}

    def fwd():
        if saved:
            m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], gu, dn, w.N, w.Z,
                                    w.K, w.I, out=y, aux=aux, workspace=ws_f)
        else:
            m.moe_zc_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                             inp["w_down"], w.N, w.Z, w.K, out=y, aux=aux, workspace=ws_f)

    def bwd():
        m.moe_zc_backward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], tr, aux, dy,
                          w.N, w.Z, w.K, w.I, out=grads, workspace=ws_b)

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_step = timed(lambda: (fwd(), bwd()))
    ms_bwd = timed(bwd)
    S = int(aux["offsets"][w.N].item())
    # expert products: q, rows of dx, three weight gradients (12 d I S), plus
    # the recomputed a and u (4 d I S) unless the forward saved them
    flop_bwd = (12.0 if saved else 16.0) * w.d * w.I * S + 4.0 * w.T * w.d * w.E
    flop_fwd = 6.0 * w.d * w.I * S + 2.0 * w.T * w.d * w.E
    out = {
        "metric": "MoE-layer training step (forward + backward) tokens/s on 1 MI355X",
        "value": w.T / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulation, fp32 weight gradients)",
        "data": "synthetic (seeded Gaussian inputs and upstream gradient, random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "I": w.I, "N": w.N, "Z": w.Z,
                   "K": w.K,
                   "step": ("moe_zc_forward_packed (saving a | u) + moe_zc_backward" if saved
                            else "moe_zc_forward + moe_zc_backward (a, u recomputed)"),
                   "parallelism": "none (1 GPU)"},
        "backward_ms": ms_bwd,
        "backward_tflops": flop_bwd / (ms_bwd / 1e3) / 1e12,
        "backward_mfma_frac": flop_bwd / (ms_bwd / 1e3) / PEAK_BF16,
        "step_tflops": (flop_fwd + flop_bwd) / (ms_step / 1e3) / 1e12,
        "ffn_rows": S,
        "cpu_baseline": None,
    }
    return out


def graph_replay(step, y, replays):
    """The same step captured once in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: the step's wall time without per-launch host overhead and gaps.
    The library allocates, synchronises and memsets nothing, so the forward
    and the PID update capture as they are.  The output of the last replay is
    compared bit for bit with the eager result, and the eager run resumes with
    the same buffers afterwards (the graph is untimed context, not the value)."""
    import torch
    try:
        torch.cuda.synchronize()
        y_ref = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(replays):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        same = bool(torch.equal(y, y_ref))
        del g
        return {"ms_per_step": (t1 - t0) * 1e3 / replays, "replays": replays,
                "bitwise_equal_to_eager": same}
    except Exception as e:  # a failed capture is reported, not fatal
        torch.cuda.synchronize()
        return {"error": f"{type(e).__name__}: {e}"[:300]}


def forward_workload(args, w, dev, precision="bf16", layout="packed", steps=20, warmup=5,
                     n_cpu=0, keep_inputs=False, fp8_down=False):
    """Time the forward of workload ``w`` as configured (its own bias on every
    timed step) plus one PID step from that routing, each timed step starting
    from the configured bias and zero PID state.  Returns a dict of results
    (and the inputs when ``keep_inputs``, for the CPU baseline)."""
    import numpy as np
    import torch

    import mixture_experts_layer_bias_amd as m
    from workloads import make_inputs

    inp = make_inputs(w, device=dev)
    dt = inp["x"].dtype
    es = inp["x"].element_size()
    fp8 = precision == "fp8"
    need = (m.moe_zc_workspace_size_fp8(w.T, w.d, w.I, w.N, w.Z, w.K) if fp8
            else m.moe_zc_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K, dt))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, dev, keys=("loads", "offsets"))
    y = torch.empty(w.T, w.d, dtype=dt, device=dev)
    bias0 = inp["bias"]                      # the configured bias: never modified
    bias_pid = bias0.clone()
    pid = m.PidState(w.E, dev, kp=0.5, ki=0.5, kd=0.0)
    target = torch.full((w.E,), w.T * w.K / w.E, dtype=torch.float32, device=dev)
    # host copies of the experts the CPU baseline evaluates
    cpu_weights = [(inp["w_gate"][e].cpu(), inp["w_up"][e].cpu(), inp["w_down"][e].cpu())
                   for e in range(min(n_cpu, w.N))]
    packed = layout == "packed" and w.dtype == "bf16"
    if packed:
        gu, dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        if fp8 and fp8_down:
            gu, dn = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"], inp["w_down"])
        elif fp8:
            gu = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"])
        torch.cuda.synchronize()
        for k in ("w_gate", "w_up", "w_down"):
            inp[k] = None
        torch.cuda.empty_cache()

    def forward(bias, events=None):
        if fp8:
            m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], bias, gu, dn, w.N, w.Z, w.K,
                                        w.I, residual=inp["residual"], out=y, aux=aux,
                                        workspace=ws, events=events, down_fp8=fp8_down)
        elif packed:
            m.moe_zc_forward_packed(inp["x"], inp["w_router"], bias, gu, dn, w.N, w.Z, w.K, w.I,
                                    residual=inp["residual"], out=y, aux=aux, workspace=ws,
                                    events=events)
        else:
            m.moe_zc_forward(inp["x"], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                             inp["w_down"], w.N, w.Z, w.K, residual=inp["residual"], out=y,
                             aux=aux, workspace=ws, events=events)

    def pid_step():
        # one bias update from the configured routing: state restored first
        bias_pid.copy_(bias0)
        pid.e_prev.zero_()
        pid.e_prev2.zero_()
        m.moe_zc_bias_update(aux["loads"], target, bias_pid, pid)

    def step(events=None, pid_ev=None):
        forward(bias0, events)
        if pid_ev:
            pid_ev[0].record()
        pid_step()
        if pid_ev:
            pid_ev[1].record()

    def ffn_stats(ld):
        f = ld[: w.N].astype(np.float64)
        return {"ffn_per_token": float(f.sum() / w.T),
                "max_over_mean_ffn_load": float(f.max() / f.mean()) if f.sum() > 0 else None}

    for _ in range(warmup):
        step()
    events = [m.StageEvents() for _ in range(steps)]
    pid_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i], pid_evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    stage = {k: 0.0 for k in m.STAGE_NAMES}
    for ev in events:
        for k, v in ev.stage_ms().items():
            stage[k] += v / steps
    pid_ms = sum(a.elapsed_time(b) for a, b in pid_evs) / steps
    loads = aux["loads"].cpu().numpy()
    S = int(aux["offsets"][w.N].item())
    touched = int((loads[: w.N] > 0).sum())

    graph = None if getattr(args, "no_graph", False) else graph_replay(step, y, steps)
    power = power_probe(step) if getattr(args, "_power_probe", False) else None
    # untimed: routing after the one PID step of the timed steps ...
    before = ffn_stats(loads)
    forward(bias_pid)
    after = ffn_stats(aux["loads"].cpu().numpy())
    # ... and a separate closed loop over repeated batches (bias carried)
    bias_cl = bias0.clone()
    pid_cl = m.PidState(w.E, dev, kp=0.5, ki=0.5, kd=0.0)
    loop = []
    for _ in range(args.closed_loop_steps):
        forward(bias_cl)
        loop.append(ffn_stats(aux["loads"].cpu().numpy()))
        m.moe_zc_bias_update(aux["loads"], target, bias_cl, pid_cl)
    torch.cuda.synchronize()

    alg = algorithmic(w, S, touched, es, fp8, fp8_down)
    flop_act = 2.0 * w.T * w.d * w.E + 6.0 * w.d * w.I * S
    t_step = ms_per_step / 1e3
    gemm_s = (stage["gemm_gate_up_swiglu"] + stage["gemm_down"]) / 1e3
    t_ideal = (4.0 * w.d * w.I * S / (PEAK_FP8 if fp8 else PEAK_BF16)
               + 2.0 * w.d * w.I * S / (PEAK_FP8 if fp8_down else PEAK_BF16))
    stage_roof = {}
    for k, v in alg.items():
        ts = stage[k] / 1e3
        if ts <= 0:
            continue
        entry = {"ms": round(stage[k], 4), "GB/s": round(v["bytes"] / ts / 1e9, 1),
                 "hbm_frac": round(v["bytes"] / ts / PEAK_HBM, 4)}
        if "flop" in v:
            pk = PEAK_FP8 if ((fp8 and k == "gemm_gate_up_swiglu") or
                              (fp8_down and k == "gemm_down")) else PEAK_BF16
            entry["TFLOP/s"] = round(v["flop"] / ts / 1e12, 1)
            entry["mfma_frac"] = round(v["flop"] / ts / pk, 4)
        stage_roof[k] = entry
    for k in ("chunk_hist", "scan"):
        stage_roof[k] = {"ms": round(stage[k], 4)}
    stage_roof["pid"] = {"ms": round(pid_ms, 4)}
    res = {
        "workload": w.name,
        "precision": (("fp8 gate/up + fp8 down" if fp8_down else "fp8 gate/up") if fp8
                      else w.dtype),
        "expert_weights": "packed" if packed else "row-major",
        "T": w.T, "d": w.d, "I": w.I, "N": w.N, "Z": w.Z, "K": w.K,
        "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "tokens_per_s": w.T / t_step,
        "activated_tflops": flop_act / t_step / 1e12,
        "activated_mfma_frac": flop_act / t_step / PEAK_BF16,
        "grouped_gemm_mfma_frac": (t_ideal / gemm_s) if (gemm_s > 0 and S > 0) else None,
        "ffn_rows": S, "ffn_experts_per_token": S / w.T, "touched_experts": touched,
        "stages": stage_roof,
        "one_pid_step": {"gains": [pid.kp, pid.ki, pid.kd], "target": "uniform T*K/E",
                         "routing_before": before, "routing_after": after},
        "closed_loop": {"steps": args.closed_loop_steps, "first": loop[0] if loop else None,
                        "last": loop[-1] if loop else None},
        "power": power,
        "graph": graph,
        "_alg": alg, "_stage_ms": stage, "_S": S, "_touched": touched, "_es": es,
    }
    if keep_inputs:
        res["_inp"] = inp
        res["_cpu_weights"] = cpu_weights
    return res


def roofline_of(res, fp8, peaks):
    """Roofline entry of the dominant kernel (gate/up + SwiGLU) of one run."""
    dom = "gemm_gate_up_swiglu"
    a = res["_alg"][dom]
    t_dom = res["_stage_ms"][dom] / 1e3
    peak_dom = PEAK_FP8 if fp8 else PEAK_BF16   # a contraction against its own dtype's peak
    t_b, t_f = a["bytes"] / PEAK_HBM, a["flop"] / peak_dom
    if t_b >= t_f:
        roof = {"bound": "hbm", "achieved": a["bytes"] / t_dom / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": a["flop"] / t_dom / 1e12, "peak": peak_dom / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if peaks:  # the same achieved rate against what the box reaches on a read stream / dense GEMM
        ref = peaks["hbm_read_GBps"] if roof["bound"] == "hbm" else (
            None if fp8 else peaks["bf16_gemm_TFLOPs"])
        roof["frac_of_measured"] = roof["achieved"] / ref if ref else None
    roof["kernel"] = dom
    roof["avg_launch_ms"] = res["_stage_ms"][dom]
    roof["algorithmic_bytes"] = a["bytes"]
    return roof


def public(res):
    return {k: v for k, v in res.items() if not k.startswith("_")}


# the other workloads timed after the headline one, in the same run
EXTRA = (("tiny", False, False), ("mid", False, False), ("decode", False, False),
         ("skew", False, False), ("prefill", True, False), ("prefill", True, True),
         ("decode", True, True))
TRAINING = ("prefill", "skew")
TRAINING_KEYS = ("metric", "value", "unit", "steps", "warmup", "ms_per_step", "config",
                 "backward_ms", "backward_tflops", "backward_mfma_frac", "step_tflops",
                 "ffn_rows")


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU only; the multi-GPU path (expert "
              "sharding with all-to-all) is not built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import get_workload

    w = get_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.which == "backward":
        print(json.dumps(bench_backward(args, w, dev)))
        return
    fp8 = args.precision == "fp8"
    if fp8 and (w.dtype != "bf16" or args.layout != "packed"):
        print("bench.py: --precision fp8 needs a bf16 workload and packed weights", file=sys.stderr)
        sys.exit(2)
    peaks = None if args.no_peak_probe else measured_peaks(dev)
    n_cpu = 0 if args.no_cpu_baseline else min(args.cpu_experts, w.N)
    if args.fp8_down and not fp8:
        print("bench.py: --fp8-down needs --precision fp8", file=sys.stderr)
        sys.exit(2)
    args._power_probe = not args.no_power_probe
    print(f"bench.py: timing {w.name} (headline)", file=sys.stderr, flush=True)
    res = forward_workload(args, w, dev, args.precision, args.layout, args.steps, args.warmup,
                           n_cpu=n_cpu, keep_inputs=not args.no_cpu_baseline,
                           fp8_down=args.fp8_down)
    args._power_probe = False
    roof = roofline_of(res, fp8, peaks)
    # the committed counter summary covers the bf16 kernel only
    roof["traffic"] = None if fp8 else counter_traffic()
    cpu = None
    if not args.no_cpu_baseline:
        print("bench.py: timing the oracle on the host cores", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, res["_inp"], args.cpu_experts, res["_cpu_weights"])
    res.pop("_inp", None)
    res.pop("_cpu_weights", None)
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra_workloads:
        for name, x8, d8 in EXTRA:
            if name == w.name and x8 == fp8 and d8 == (fp8 and args.fp8_down):
                continue
            wx = get_workload(name)
            steps = max(3, min(args.steps, 20))
            print(f"bench.py: timing {name}{' fp8' if x8 else ''}{' fp8-down' if d8 else ''}",
                  file=sys.stderr, flush=True)
            rx = forward_workload(args, wx, dev, "fp8" if x8 else "bf16", "packed", steps,
                                  min(args.warmup, 3), fp8_down=d8)
            rx["roofline_gate_up"] = {k: v for k, v in roofline_of(rx, x8, None).items()
                                      if k in ("bound", "achieved", "peak", "unit", "frac")}
            extra[name + ("_fp8" if x8 else "") + ("_fp8down" if d8 else "")] = public(rx)
            del rx
            torch.cuda.empty_cache()
        # the training step (forward saving a | u, then the backward) of the
        # prefill and skewed layers, as `--pass backward` times it
        for name in TRAINING:
            print(f"bench.py: timing the training step of {name}", file=sys.stderr, flush=True)
            rt = bench_backward(args, get_workload(name), dev, steps=max(3, min(args.steps, 10)),
                                warmup=min(args.warmup, 3))
            extra["training_" + name] = {k: rt[k] for k in TRAINING_KEYS}
            del rt
            torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("fp8-e4m3 block-scaled gate/up and down" if args.fp8_down else
                   "fp8-e4m3 block-scaled gate/up + bf16") if fp8
                  else ("bf16" if w.dtype == "bf16" else "f32")),
        "data": "synthetic (seeded Gaussian inputs, random-init expert weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "I": w.I, "N": w.N, "Z": w.Z,
                   "K": w.K, "expert_ffn": "SwiGLU", "residual": True,
                   "step": ("moe_zc_forward_packed_fp8" if fp8 else
                            "moe_zc_forward_packed" if res["expert_weights"] == "packed"
                            else "moe_zc_forward")
                   + " with the configured bias + one moe_zc_bias_update",
                   "precision": (("gate/up and down block FP8 (E4M3, power-of-two scale "
                                  "per 32 k); router, combine bf16/fp32") if args.fp8_down else
                                 ("gate/up block FP8 (E4M3, power-of-two scale per 32 k); "
                                  "router, down, combine bf16/fp32") if fp8 else "bf16"),
                   "expert_weights": res["expert_weights"],
                   "parallelism": "none (1 GPU)"},
        "activated_tflops": res["activated_tflops"],
        "activated_mfma_frac": res["activated_mfma_frac"],
        "grouped_gemm_mfma_frac": res["grouped_gemm_mfma_frac"],
        "ffn_rows": res["ffn_rows"],
        "ffn_experts_per_token": res["ffn_experts_per_token"],
        "touched_experts": res["touched_experts"],
        "stages": res["stages"],
        "one_pid_step": res["one_pid_step"],
        "closed_loop": res["closed_loop"],
        "power": res["power"],
        "graph": res["graph"],
        "measured_peaks": peaks,
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": extra,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
