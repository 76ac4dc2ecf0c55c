"""Throughput of the Gated DeltaNet token mixer on one MI355X.

A step is one pass of the prefill hot path over one synthetic layer input:
gdn_conv1d (causal conv + SiLU over [q|k|v]) then gdn_prefill (chunked gated
delta rule), inputs already resident in HBM.  The default workload is the
9B-shaped layer (B=1, T=8192, 32 QK / 32 V heads, d=128, chunk 64).  The line
also carries the decode leg: gdn_decode_step on the 27B-shaped batch of 256
sequences x 48 V heads with a bf16 state, 64 consecutive steps.

The `backward` object times the training backward of the same layer:
gdn_prefill_backward then gdn_conv1d_backward, with the forward's conv output
and the output gradient resident.

Prints ONE JSON line.  `value` is prefill tokens/s/layer (conv + prefill).
`roofline` is for the dominant kernel (the prefill kernel): algorithmic
FLOPs per launch / its average duration from HIP events on the stream it
runs on.  `cpu_baseline` is the fp64 oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "GDN prefill tokens/s/layer (%MFMA peak); decode steps/s (%HBM BW), 1 MI355X"


def prefill_flops_per_token(cfg):
    """Algorithmic FLOPs per token of the chunked form: per V head the W/U-sized
    C x C products (2 C d_k + 4 C d_v: T-apply, intra-chunk output) and the
    d_k x d_v state products (6 d_k d_v: S k, S q, state update), plus the two
    Gram matrices once per QK head (4 C d_k)."""
    C, dk, dv = cfg["chunk"], cfg["d_k"], cfg["d_v"]
    return cfg["h_v"] * (2 * C * dk + 4 * C * dv + 6 * dk * dv) + cfg["h_qk"] * 4 * C * dk


def backward_flops_per_token(cfg):
    """Contraction FLOPs per token of the chunked backward as computed (fp32):
    per V head and chunk, 22 C x C x d products (recomputed W and Ut, Pm^T dO,
    T^T dU, dPm, dT (2), T^T dW, dK^ (2), dQ^ ...), 16 C x d x d products (the
    two chains' 4, Z, dW, dO X^T, U dX'^T) and 4 C^3 (dT T^T, T^T M1), plus
    the two Gram matrices per QK head; divided by the C tokens of a chunk."""
    C, d = cfg["chunk"], cfg["d_k"]
    return cfg["h_v"] * (22 * C * d + 16 * d * d + 4 * C * C) + cfg["h_qk"] * 4 * C * d


def decode_bytes_per_step(cfg):
    """HBM bytes one decode step must move: state read + write, conv-state
    history read (W-1) and one new slot written, x, g and beta, o, conv weights."""
    N, hv, dk, dv, W = cfg["n_seqs"], cfg["h_v"], cfg["d_k"], cfg["d_v"], cfg["width"]
    C = 2 * cfg["h_qk"] * dk + hv * dv
    sb = 2 if cfg["state"] == "bf16" else 4
    return (2 * N * hv * dv * dk * sb + N * C * W * 2 + N * C * 2 + N * hv * 8 + N * hv * dv * 2
            + C * W * 2)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_token_conv1d_amd", "csrc")


def measured_traffic(summary, source):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the factor a plain copy of known
    size reads on the same counter).  None when the summary is missing or was
    taken on a different version of the kernel source."""
    import hashlib
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip().lstrip("- ")] = v.strip().strip("`")
    digest = hashlib.sha256(open(os.path.join(CSRC, source), "rb").read()).hexdigest()
    if fields.get(f"sha256 {source}") != digest or "traffic_bytes_per_launch" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def calibrate_copy(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters: profiled with the same counters as the kernels."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "launches": reps}), flush=True)


_SHARED = {}  # oracle inputs handed to forked workers without pickling


def _oracle_heads(heads):
    from oracle import gdn_oracle as orc
    s = _SHARED
    orc.gdn_layer(s["x"], s["w"], s["g"], s["b"], s["hq"], s["d"], s["hv"], s["d"], v_heads=heads)
    return len(heads)


def cpu_baseline_prefill(inp, cfg, tokens):
    """Oracle (fp64 numpy, token by token) over the first `tokens` tokens of the
    workload, all V heads, split over a process pool by V head."""
    import numpy as np
    cores = min(len(os.sched_getaffinity(0)), cfg["h_v"], 16)
    tokens = min(tokens, inp["T"])
    x = inp["x"][:tokens].double().numpy()
    w = inp["conv_weight"].double().numpy()
    g = inp["g"][:tokens].double().numpy()
    b = inp["beta"][:tokens].double().numpy()
    jobs = [list(h) for h in np.array_split(np.arange(cfg["h_v"]), cores)]
    _SHARED.update(x=x, w=w, g=g, b=b, hq=cfg["h_qk"], d=cfg["d_k"], hv=cfg["h_v"])
    ctx = mp.get_context("fork")
    t = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.map(_oracle_heads, jobs))
    dt = time.perf_counter() - t
    assert done == cfg["h_v"]
    return {"value": tokens / dt, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} of {cfg['T']} tokens, all {cfg['h_v']} V heads, conv + recurrence, "
                      f"fp64 numpy, {cores} processes split by V head; {dt:.1f} s"}


def run_prefill(name, steps, warmup, do_cpu, cpu_tokens):
    import torch
    import gdn_inputs
    import linear_attention_token_conv1d_amd as gdn

    inp = gdn_inputs.prefill_inputs(name)
    cfg = inp["cfg"]
    dev = torch.device("cuda:0")
    x = inp["x"].to(dev)
    w = inp["conv_weight"].to(dev)
    g = inp["g"].to(dev)
    beta = inp["beta"].to(dev)
    s0 = None if inp["initial_state"] is None else inp["initial_state"].to(dev)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].to(dev)
    T, hq, hv, d = inp["T"], cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    y = torch.empty_like(x)
    o = torch.empty((T, hv, d), dtype=x.dtype, device=dev)
    fs = torch.empty((inp["n_seqs"], hv, d, d), dtype=torch.float32, device=dev)
    q0, _, v0 = gdn.split_qkv(y, hq, d, hv, d)
    ws = torch.empty(max(1, gdn.prefill_workspace_size(q0, v0, inp["n_seqs"], cfg["chunk"])),
                     dtype=torch.uint8, device=dev)

    def step(ev=None):
        gdn.conv1d(x, w, None, None, cu, "silu", out=y)
        q, k, v = gdn.split_qkv(y, hq, d, hv, d)
        if ev is not None:
            ev[0].record()
        gdn.prefill(q, k, v, g, beta, s0, cu, cfg["chunk"], 1.0, True, True, o=o, final_state=fs,
                    workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    k_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    flops = prefill_flops_per_token(cfg) * T
    tflops = flops / (k_ms * 1e-3) / 1e12
    res = {
        "tokens_per_s": T / (ms * 1e-3),
        "ms_per_step": ms,
        "prefill_kernel_ms": k_ms,
        "prefill_only_tokens_per_s": T / (k_ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(f"prefill_{name}_traffic.md", "prefill.hip"),
                     "kernel": "gdn_prefill (prep_kernel, scan2_kernel; plan_kernel with cu_seqlens, join_kernel after a split scan)",
                     "flops_per_launch": flops},
        "config": {"workload": f"{name}: B={inp['n_seqs']} T={T} h_qk={hq} h_v={hv} d={d} "
                               f"chunk={cfg['chunk']} conv{cfg['width']}+SiLU, bf16 io, fp32 state",
                   "tokens": T, "h_qk": hq, "h_v": hv, "d": d, "chunk": cfg["chunk"]},
    }
    if do_cpu:
        res["cpu_baseline"] = cpu_baseline_prefill(inp, cfg, cpu_tokens)
    return res


def run_backward(name, steps, warmup, do_cpu):
    import torch
    import gdn_inputs
    import linear_attention_token_conv1d_amd as gdn

    inp = gdn_inputs.prefill_inputs(name)
    cfg = inp["cfg"]
    dev = torch.device("cuda:0")
    x = inp["x"].to(dev)
    w = inp["conv_weight"].to(dev)
    g = inp["g"].to(dev)
    beta = inp["beta"].to(dev)
    s0 = None if inp["initial_state"] is None else inp["initial_state"].to(dev)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].to(dev)
    T, hq, hv, d, N = inp["T"], cfg["h_qk"], cfg["h_v"], cfg["d_k"], inp["n_seqs"]
    y = gdn.conv1d(x, w, None, None, cu, "silu")
    q, k, v = gdn.split_qkv(y, hq, d, hv, d)
    gen = torch.Generator().manual_seed(1)
    do = torch.randn((T, hv, d), generator=gen).to(torch.bfloat16).to(dev)
    dy = torch.zeros_like(y)
    dq, dk, dv = gdn.split_qkv(dy, hq, d, hv, d)
    dg = torch.empty((T, hv), dtype=torch.float32, device=dev)
    db = torch.empty_like(dg)
    ds0 = torch.empty((N, hv, d, d), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.prefill_backward_workspace_size(q, v, N, cfg["chunk"]), dtype=torch.uint8, device=dev)
    cws = torch.empty(gdn.conv1d_backward_workspace_size(T, y.shape[1]), dtype=torch.uint8, device=dev)
    dx = torch.empty_like(x)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gdn.prefill_backward(q, k, v, g, beta, do, s0, None, cu, cfg["chunk"], 1.0, True, True, dq=dq, dk=dk,
                             dv=dv, dg=dg, dbeta=db, d_initial_state=ds0, workspace=ws)
        if ev is not None:
            ev[1].record()
        gdn.conv1d_backward(x, w, dy, None, None, cu, "silu", None, dx=dx, d_conv_state=False, workspace=cws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(evs[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    k_ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    flops = backward_flops_per_token(cfg) * T
    tflops = flops / (k_ms * 1e-3) / 1e12
    res = {"tokens_per_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "prefill_backward_ms": round(k_ms, 4),
           "roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / PEAK_F32_TFLOPS, 4),
                        "traffic": measured_traffic(f"backward_{name}_traffic.md", "backward.hip"),
                        "kernel": "gdn_prefill_backward (fp32 batched GEMMs, two chains, fused chunk-local kernel; a QK-head kernel when a QK head has several V heads)",
                        "flops_per_launch": flops},
           "config": {"workload": f"{name} backward: gdn_prefill_backward + gdn_conv1d_backward, B={N} T={T} "
                                  f"h_qk={hq} h_v={hv} d={d} chunk={cfg['chunk']}, bf16 io, fp32 arithmetic"}}
    if do_cpu:
        from oracle import gdn_oracle as orc
        tok = 1024
        h = 0
        qn, kn, vn = (t[:tok, h:h + 1].double().cpu().numpy() for t in (q, k, v))
        t0 = time.perf_counter()
        orc.gated_delta_rule_backward(qn, kn, vn, g[:tok, h:h + 1].double().cpu().numpy(),
                                      beta[:tok, h:h + 1].double().cpu().numpy(),
                                      do[:tok, h:h + 1].double().cpu().numpy(), segment=64)
        dt = (time.perf_counter() - t0) * (T / tok) * hv
        res["cpu_baseline"] = {"value": round(T / dt, 1), "unit": "tokens/s/layer", "cores": 1, "kind": "oracle",
                               "sample": f"oracle backward of V head 0 over the first {tok} tokens, fp64 numpy, "
                                         f"one process; time scaled by {T // tok} x {hv} heads"}
    return res


def run_decode(steps, warmup, do_cpu):
    import numpy as np
    import torch
    import gdn_inputs
    import linear_attention_token_conv1d_amd as gdn

    inp = gdn_inputs.decode_inputs("qwen35_27b_decode")
    cfg = inp["cfg"]
    dev = torch.device("cuda:0")
    S = inp["state"].to(dev)
    cs = inp["conv_state"].to(dev)
    w = inp["conv_weight"].to(dev)
    xs, gs, bs = inp["x"].to(dev), inp["g"].to(dev), inp["beta"].to(dev)
    N, hq, hv, d = cfg["n_seqs"], cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    o = torch.empty((N, hv, d), dtype=torch.bfloat16, device=dev)
    nsteps = xs.shape[0]
    # untimed: at least one full pass of the 64 steps (the clocks settle over
    # the first few dozen launches)
    for i in range(max(warmup, nsteps)):
        gdn.decode_step(xs[i % nsteps], gs[i % nsteps], bs[i % nsteps], S, hq, hv, d, conv_weight=w,
                        conv_state=cs, o=o)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(nsteps):
        gdn.decode_step(xs[i], gs[i], bs[i], S, hq, hv, d, conv_weight=w, conv_state=cs, o=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / nsteps
    nbytes = decode_bytes_per_step(cfg)
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {"value": 1e3 / ms, "unit": "steps/s", "tokens_per_s": N * 1e3 / ms, "ms_per_step": ms,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic("decode_qwen35_27b_decode_traffic.md", "decode.hip"),
                        "kernel": "decode_kernel<bf16,bf16,128>", "bytes_per_launch": nbytes},
           "config": {"workload": f"qwen35_27b_decode: {N} sequences x 1 token, h_qk={hq} h_v={hv} d={d}, "
                                  f"bf16 state, conv4+SiLU, {nsteps} consecutive steps"}}
    if do_cpu:
        from oracle import gdn_oracle as orc
        sample = 8
        st = inp["state"][:sample].double().numpy()
        ct = inp["conv_state"][:sample].double().numpy()
        wn = inp["conv_weight"].double().numpy()
        t = time.perf_counter()
        for i in range(4):
            _, st, ct = orc.decode_step(inp["x"][i, :sample].double().numpy(), wn,
                                        inp["g"][i, :sample].double().numpy(),
                                        inp["beta"][i, :sample].double().numpy(), st, ct, hq, d, hv, d)
        dt = (time.perf_counter() - t) / 4 * (N / sample)
        res["cpu_baseline"] = {"value": 1.0 / dt, "unit": "steps/s", "cores": 1, "kind": "oracle",
                               "sample": f"{sample} of {N} sequences x 4 steps, fp64 numpy, one process; "
                                         f"time scaled by {N // sample}"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen35_9b_prefill",
                    choices=["qwen35_9b_prefill", "qwen35_27b_prefill", "qwen35_27b_varlen"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the mixer shards by (sequence, V head) with no "
              "exchange, so there is no multi-GPU step to time here.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    pre = run_prefill(args.workload, args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_tokens)
    line = {"metric": METRIC, "value": round(pre["tokens_per_s"], 1), "unit": "tokens/s/layer",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(pre["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": pre["config"], "roofline": pre["roofline"],
            "prefill_kernel_ms": round(pre["prefill_kernel_ms"], 4),
            "prefill_only_tokens_per_s": round(pre["prefill_only_tokens_per_s"], 1)}
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
    if not args.no_decode:
        line["decode"] = run_decode(args.steps, args.warmup, not args.no_cpu_baseline)
    if not args.no_backward:
        line["backward"] = run_backward(args.workload, args.steps, args.warmup, not args.no_cpu_baseline)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
