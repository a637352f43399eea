"""Throughput of the DeepSeekMoE layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full layer forward (router, dispatch, grouped SwiGLU expert
GEMMs with the shared experts in the same launches, combine) over one batch
of seeded synthetic hidden states, with every input already resident in HBM.
The layer backward (all gradients, routing recomputed) is timed beside it.
The default workload is the 16B-model-shaped prefill layer in bfloat16
(T=8192 tokens, d=2048, 64 routed + 2 shared experts, top-6, intermediate
1408).  The decode-shaped batch (T=64, same layer) is timed beside it.
Before each prefill workload's W warm-up and K timed steps, untimed forwards
run for SETTLE_S seconds of GPU time (reported as "settle"): the inputs are
generated on the host while the GPU idles, and its clocks need longer than a
few steps to reach their level under this load.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (MFMA / vector)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
SETTLE_S = 0.25               # untimed forwards before each prefill timed pass (GPU time)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="moe16b_prefill_bf16")
    ap.add_argument("--decode-workload", default="moe16b_decode_bf16")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the layer backward beside the forward")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the layer backward of the workload (for profiling runs)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--other-workloads", default="moe2b_bf16:4096,moe145b_skewed_bf16:2048",
                    help="comma-separated NAME:CPU_TOKENS of further workloads timed beside the "
                         "main one (CPU_TOKENS: the oracle's token sample); empty for none")
    ap.add_argument("--sweep", action="store_true",
                    help="granularity sweep instead of the benchmark line: the same layer "
                         "cut into m in {1,2,4,8} times finer experts, K_s in {0,1} shared, at "
                         "equal parameters and FLOPs; prints one JSON line per configuration")
    ap.add_argument("--profile-mode", action="store_true",
                    help="for hardware-counter runs: a 1 GiB device copy (calibration) and two "
                         "layer forwards of the workload, nothing else")
    args = ap.parse_args()
    args.other_workloads = [(n, int(c)) for n, c in
                            (x.split(":") for x in args.other_workloads.split(",") if x)]
    return args


def profile_mode(args):
    """Short, fixed sequence for rocprofv3 counter passes: torch's copy kernel moving a known
    1 GiB (reads 1 GiB, writes 1 GiB) three times, then two forwards of the workload."""
    import torch

    import moe_inputs
    import mixture_experts_ffn_fp32_amd as mx

    dev = torch.device("cuda:0")
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    inp = moe_inputs.make(args.workload)
    t = upload(inp, dev)
    w = inp.w
    for _ in range(2):
        mx.layer_forward(t["u"], t["E"], t["Wr"], t["Ws"], w.N, w.K, w.K_s, t["bias"])
    torch.cuda.synchronize()
    print(json.dumps({"profile_mode": w.name, "copy_bytes_each_way": 1 << 30}), flush=True)


def upload(inp, device):
    import numpy as np
    import torch

    def dev(raw):
        t = torch.from_numpy(np.ascontiguousarray(raw))
        if inp.w.dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(device)

    w = inp.w
    b = inp.gate_bias()
    return dict(u=dev(inp.u_raw()), E=dev(inp.E_gate_raw()), Wr=dev(inp.routed_all_raw(threads=16)),
                Ws=dev(inp.shared_all_raw()) if w.K_s else None,
                bias=None if b is None else torch.from_numpy(b).to(device))


def time_layer(mx, t, w, steps, warmup, stage_timing, per_step_events=False):
    """Warm up, then time exactly `steps` forwards between two synchronisations.
    stage_timing: False, True (every stage timed) or a list of stage names (those stages
    only); the library times a stage with events carried by its own kernel launches.
    per_step_events: an event between consecutive steps as well (per-step times for the
    median and percentiles; each is a marker in the stream, so the pass that gives the
    headline time goes without them).
    Returns (total ms, [ms of each step] or None, {stage: (ms, launches)})."""
    import torch

    I = t["Wr"].numel() // (3 * w.N * w.d)
    ws = torch.empty(mx.workspace_size(w.T, w.d, I, w.N, w.K, w.K_s, 1 if w.dtype == "bf16" else 0),
                     dtype=torch.uint8, device=t["u"].device)
    h = torch.empty_like(t["u"])
    args = (t["u"], t["E"], t["Wr"], t["Ws"], w.N, w.K, w.K_s, t["bias"])
    for _ in range(warmup):
        mx.layer_forward(*args, out=h, workspace=ws)
    torch.cuda.synchronize()
    mx.timing_read()                       # drop anything recorded before
    mx.timing_enable(bool(stage_timing),
                     None if isinstance(stage_timing, bool) else list(stage_timing))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        mx.layer_forward(*args, out=h, workspace=ws)
        if per_step_events or i + 1 == steps:
            ev[i + 1].record()
    torch.cuda.synchronize()
    mx.timing_enable(False)
    stages = mx.timing_read()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)] if per_step_events else None
    return ev[0].elapsed_time(ev[steps]), per_step, stages


def settle(mx, t, w, seconds):
    """Untimed forwards for about `seconds` of GPU time before a timed pass: the inputs
    were just generated on the host while the GPU idled, and its clocks take longer to
    reach their level under this load than a few warm-up steps (a fixed time, not a step
    count, so a short --warmup still times the steady state).  Returns the steps run."""
    import torch

    if seconds <= 0:
        return 0
    I = t["Wr"].numel() // (3 * w.N * w.d)
    ws = torch.empty(mx.workspace_size(w.T, w.d, I, w.N, w.K, w.K_s, 1 if w.dtype == "bf16" else 0),
                     dtype=torch.uint8, device=t["u"].device)
    h = torch.empty_like(t["u"])
    args = (t["u"], t["E"], t["Wr"], t["Ws"], w.N, w.K, w.K_s, t["bias"])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, done, batch = 0, 0.0, 4
    while done < seconds * 1e3:
        e0.record()
        for _ in range(batch):
            mx.layer_forward(*args, out=h, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)
        n += batch
        batch = min(batch * 2, 64)
    return n


def step_stats(per_step):
    """Median, 10th and 90th percentile of the per-step times (ms)."""
    import numpy as np

    q = np.percentile(np.asarray(per_step), [50, 10, 90])
    return {"median": round(float(q[0]), 4), "p10": round(float(q[1]), 4),
            "p90": round(float(q[2]), 4)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gemm_rooflines(w, stages, peak):
    """TFLOP/s and fraction of peak of both expert GEMMs from the per-stage event pairs."""
    out = {}
    for key, per_pair in (("expert_gemm1_swiglu", 4.0), ("expert_gemm2_down", 2.0)):
        ms, n = stages[key]
        if not n:
            continue
        fl = per_pair * w.d * w.I * w.T * (w.K + w.K_s)
        tf = fl / (ms / n / 1e3) / 1e12
        out[key] = {"launch_ms": round(ms / n, 4), "tflops": round(tf, 2),
                    "frac": round(tf / peak, 4)}
    return out


def time_backward(mx, t, w, steps, warmup):
    """Warm up, then time exactly `steps` layer backwards (routing recomputed, every
    gradient written) between two synchronisations; returns elapsed ms."""
    import torch

    g = torch.Generator(device=t["u"].device)
    g.manual_seed(w.seed + 7)
    dh = torch.randn(t["u"].shape, generator=g, device=t["u"].device, dtype=t["u"].dtype)
    I = t["Wr"].numel() // (3 * w.N * w.d)
    ws = torch.empty(mx.backward_workspace_size(w.T, w.d, I, w.N, w.K, w.K_s,
                                                1 if w.dtype == "bf16" else 0),
                     dtype=torch.uint8, device=t["u"].device)
    args = (t["u"], t["E"], t["Wr"], t["Ws"], w.N, w.K, w.K_s, dh, t["bias"])
    for _ in range(warmup):
        out = mx.layer_backward(*args, workspace=ws)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        out = mx.layer_backward(*args, workspace=ws)
    stop.record()
    torch.cuda.synchronize()
    del out, ws
    return start.elapsed_time(stop)


def backward_flops(w, I):
    """MFMA FLOPs of one backward: per expert slot the recomputed gate/up product (4dI),
    dP (2dI), dx (4dI), dW_down (2dI), dW_gate and dW_up (4dI); dE_gate 2Nd per token."""
    return 16.0 * w.d * I * w.T * (w.K + w.K_s) + 2.0 * w.N * w.d * w.T


def experts_hit(mx, t, w):
    """Distinct routed experts selected in the batch (the decode weights actually streamed)."""
    idx, _, _ = mx.route(t["u"], t["E"], w.K, t["bias"])
    return int(idx.unique().numel())


def cpu_baseline(inp, n_tokens):
    """The float64 oracle, as it stands, on the first n_tokens tokens of the workload
    (the router over those tokens, each selected expert over its tokens among them)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    w = inp.w
    routed_raw = inp.routed_all_raw(threads=16)
    shared_raw = inp.shared_all_raw()
    f32 = (lambda r: (r.astype(np.uint32) << 16).view(np.float32)) if w.dtype == "bf16" else (lambda r: r)
    routed = lambda e: inp.split_block(f32(routed_raw[e]))   # noqa: E731
    shared = lambda j: inp.split_block(f32(shared_raw[j]))   # noqa: E731
    tokens = np.arange(min(n_tokens, w.T))
    t0 = time.perf_counter()
    oracle.moe_forward_tokens(inp.u_f32(), inp.E_gate_f32(), routed, shared, w.N, w.K, w.K_s,
                              inp.gate_bias(), tokens)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(len(tokens) / dt, 1), "unit": "tokens/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {len(tokens)} of {w.T} tokens of {w.name} (router over the sample, "
                      f"all experts' weights decoded), {dt:.2f} s wall"}


def sweep(args):
    """Granularity sweep (equal expert parameters and FLOPs per token): one JSON line per
    configuration.  Inputs are drawn on the GPU (torch's seeded generator: u ~ N(0,1),
    gate vectors and weights ~ N(0, sigma^2), bf16); their values only set the routing,
    which is near-uniform as in the main workload."""
    import torch

    import moe_inputs
    import mixture_experts_ffn_fp32_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mx.load_library()
    for m, ks in moe_inputs.GRANULARITY_SWEEP:
        w = moe_inputs.granularity(m, ks)
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed)
        bf = torch.bfloat16
        t = {"u": torch.randn(w.T, w.d, generator=g, device=dev, dtype=bf),
             "E": torch.randn(w.N, w.d, generator=g, device=dev, dtype=bf) * w.sigma,
             "Wr": torch.randn(w.N * 3 * w.I * w.d, generator=g, device=dev, dtype=bf) * w.sigma,
             "Ws": (torch.randn(w.K_s * 3 * w.I * w.d, generator=g, device=dev, dtype=bf) * w.sigma
                    if w.K_s else None),
             "bias": None}
        settle(mx, t, w, SETTLE_S)
        ms, _, _ = time_layer(mx, t, w, args.steps, args.warmup, False)
        _, per_step, _ = time_layer(mx, t, w, args.steps, 1, False, per_step_events=True)
        _, _, stages = time_layer(mx, t, w, args.steps, 1, True)
        step = ms / args.steps / 1e3
        tflops = w.flops_per_token() * w.T / step / 1e12
        print(json.dumps({
            "sweep": w.name, "m": m, "shared_experts": ks, "routed_experts": w.N, "top_k": w.K,
            "intermediate": w.I, "T": w.T, "d": w.d, "dtype": w.dtype,
            "ms_per_step": round(step * 1e3, 4), "step_ms": step_stats(per_step),
            "tokens_per_s": round(w.T / step, 1),
            "layer_tflops": round(tflops, 2), "layer_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "stage_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in stages.items()}}), flush=True)
        del t
        torch.cuda.empty_cache()


def backward_only(args):
    import torch

    import moe_inputs
    import mixture_experts_ffn_fp32_amd as mx

    dev = torch.device("cuda:0")
    inp = moe_inputs.make(args.workload)
    w = inp.w
    t = upload(inp, dev)
    ms = time_backward(mx, t, w, args.steps, args.warmup) / args.steps
    fl = backward_flops(w, w.I)
    print(json.dumps({"backward": w.name, "ms_per_step": round(ms, 4),
                      "tflops": round(fl / (ms / 1e3) / 1e12, 2)}), flush=True)


def traffic_record(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary (profiles/traffic.json),
    if it was taken on the current source of the kernel it names (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key)
    if not rec:
        return None
    src = open(os.path.join(ROOT, "mixture_experts_ffn_fp32_amd", "csrc", rec["source"]), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("bytes_per_launch")


def other_workload(mx, name, steps, warmup, cpu_tokens):
    """One more prefill-sized workload, reported beside the main line: tokens/s, the step
    time's median and percentiles, the layer's and each GEMM's fraction of bf16 MFMA
    peak, the stage times, and the oracle on a token sample (None: no CPU baseline)."""
    import torch

    import moe_inputs

    inp = moe_inputs.make(name)
    w = inp.w
    t = upload(inp, torch.device("cuda:0"))
    settle(mx, t, w, SETTLE_S)
    ms, _, _ = time_layer(mx, t, w, steps, warmup, False)
    _, per_step, _ = time_layer(mx, t, w, steps, 1, False, per_step_events=True)
    _, _, stages = time_layer(mx, t, w, steps, 1, True)
    del t
    torch.cuda.empty_cache()
    step = ms / steps
    tf = w.flops_per_token() * w.T / (step / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    out = {"workload": w.name, "T": w.T, "d": w.d, "routed_experts": w.N, "top_k": w.K,
           "shared_experts": w.K_s, "intermediate": w.I, "dtype": w.dtype,
           "ms_per_step": round(step, 4), "step_ms": step_stats(per_step),
           "tokens_per_s": round(w.T / (step / 1e3), 1), "layer_tflops": round(tf, 2),
           "layer_mfma_frac": round(tf / peak, 4), "gemms": gemm_rooflines(w, stages, peak),
           "stage_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in stages.items() if v[1]}}
    if cpu_tokens:
        out["cpu_baseline"] = cpu_baseline(inp, cpu_tokens)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.profile_mode:
        return profile_mode(args)
    if args.sweep:
        return sweep(args)
    if args.backward_only:
        return backward_only(args)
    import torch

    import moe_inputs
    import mixture_experts_ffn_fp32_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mx.load_library()

    # ---- main workload
    inp = moe_inputs.make(args.workload)
    w = inp.w
    t = upload(inp, dev)
    settled = settle(mx, t, w, SETTLE_S)
    # the timed steps carry events around GEMM1 only (its launch duration for the
    # roofline); the per-stage breakdown comes from a second pass with every stage
    ms, _, g1_stage = time_layer(mx, t, w, args.steps, args.warmup, ["expert_gemm1_swiglu"])
    _, per_step, _ = time_layer(mx, t, w, args.steps, 1, False, per_step_events=True)
    _, _, stages = time_layer(mx, t, w, args.steps, 1, True)
    ms_step = ms / args.steps
    value = w.T * args.steps / (ms / 1e3)
    flops_step = w.flops_per_token() * w.T
    g1_ms, g1_n = g1_stage["expert_gemm1_swiglu"]
    g1_flops = 4.0 * w.d * w.I * w.T * (w.K + w.K_s)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    g1_tflops = g1_flops / (g1_ms / g1_n / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": "expert_gemm1_swiglu", "achieved": round(g1_tflops, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(g1_tflops / peak, 4),
                "traffic": traffic_record(f"{w.name}:expert_gemm1_swiglu"),
                "launch_ms": round(g1_ms / g1_n, 4),
                "algorithmic_flops_per_launch": g1_flops}
    stage_ms = {k: round(v[0] / max(v[1], 1), 4) for k, v in stages.items()}
    layer_tflops = flops_step / (ms_step / 1e3) / 1e12
    backward = None
    if not args.no_backward:
        bsteps = max(1, args.steps // 2)
        bms = time_backward(mx, t, w, bsteps, 1) / bsteps
        bflops = backward_flops(w, w.I)
        backward = {"workload": w.name, "ms_per_step": round(bms, 4),
                    "tokens_per_s": round(w.T / (bms / 1e3), 1), "steps": bsteps,
                    "mfma_flops": bflops, "tflops": round(bflops / (bms / 1e3) / 1e12, 2),
                    "mfma_frac": round(bflops / (bms / 1e3) / 1e12 / peak, 4)}
    del t
    torch.cuda.empty_cache()

    # ---- decode-shaped batch (HBM bound): weights of every hit expert streamed once
    decode = None
    if args.decode_workload:
        dinp = moe_inputs.make(args.decode_workload)
        dw = dinp.w
        dt_ = upload(dinp, dev)
        dms, _, _ = time_layer(mx, dt_, dw, args.decode_steps, 10, False)
        _, dper, _ = time_layer(mx, dt_, dw, args.decode_steps, 2, False, per_step_events=True)
        _, _, dstages = time_layer(mx, dt_, dw, args.decode_steps, 2, True)
        hit = experts_hit(mx, dt_, dw)
        es = 2 if dw.dtype == "bf16" else 4
        dbytes = ((hit + dw.K_s) * 3 * dw.d * dw.I * es + dw.N * dw.d * es
                  + 2 * dw.T * dw.d * es + dw.T * dw.K * 8)
        dstep = dms / args.decode_steps / 1e3
        decode = {"workload": dw.name, "tokens_per_s": round(dw.T / dstep, 1),
                  "ms_per_step": round(dstep * 1e3, 4), "step_ms": step_stats(dper),
                  "experts_hit": hit,
                  "algorithmic_bytes": dbytes, "hbm_GBs": round(dbytes / dstep / 1e9, 1),
                  "hbm_frac": round(dbytes / dstep / 1e9 / PEAK_HBM_GBS, 4),
                  # counter-measured HBM bytes of the two expert GEMMs (rocprofv3 FETCH_SIZE +
                  # WRITE_SIZE, profiles/traffic.json; null once their source has changed)
                  "gemm_traffic": {k: traffic_record(f"{dw.name}:{k}")
                                   for k in ("expert_gemm1_swiglu", "expert_gemm2_down")},
                  "stage_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in dstages.items()
                               if v[1]}}
        del dt_
        torch.cuda.empty_cache()

    # ---- the other prefill-sized workloads (2B-class, 145B-class with skewed routing)
    others = {}
    for name, cpu_tokens in ((n, c) for n, c in args.other_workloads if n):
        others[name] = other_workload(mx, name, args.steps, args.warmup,
                                      None if args.no_cpu_baseline else cpu_tokens)

    cpu = None if args.no_cpu_baseline else cpu_baseline(inp, args.cpu_sample_tokens)

    line = {
        "metric": "MoE-layer tokens/s (16B shape, bf16) + % bf16 MFMA peak / % HBM peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"seconds": SETTLE_S, "steps": settled},
        "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "routed_experts": w.N, "top_k": w.K,
                   "shared_experts": w.K_s, "intermediate": w.I, "accumulate": "f32",
                   "global_batch": w.T, "parallelism": "single GPU"},
        "step_ms": step_stats(per_step),
        "layer_tflops": round(layer_tflops, 2),
        "layer_mfma_frac": round(layer_tflops / peak, 4),
        "gemms": gemm_rooflines(w, stages, peak),
        "stage_ms": stage_ms,
        "roofline": roofline,
        "decode": decode,
        "workloads": others,
        "backward": backward,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
