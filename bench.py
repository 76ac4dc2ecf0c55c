"""Throughput of the Gated DeltaNet token mixer on one MI355X.

A step is one pass of the prefill hot path over one synthetic layer input:
gdn_conv1d (causal conv + SiLU over [q|k|v]) then gdn_prefill (chunked gated
delta rule), inputs already resident in HBM.  The headline workload is the
27B-shaped varlen pack: 8 sequences, log-uniform lengths in [4096, 65536],
262,144 tokens, 16 QK / 48 V heads, d = 128, chunk 64 -- the largest
configuration that fits one GPU.  The 9B-shaped layer (T = 8192, 32/32 heads)
and the 27B-shaped single sequence (T = 65,536) are timed the same way as
extra keys.  Between timed steps a 1 GiB scratch write flushes the 256 MB
last-level cache (outside the timed brackets), so no step finds the previous
step's data on chip.

The line also carries the decode legs: gdn_decode_step on the 27B-shaped
batch of 256 sequences x 48 V heads, 64 consecutive steps, with the conv
state as a ring, for a bf16 state and for an fp32 state, and the training
backward of the 9B layer (gdn_prefill_backward then gdn_conv1d_backward).

Prints ONE JSON line.  `value` is prefill tokens/s/layer (conv + prefill) on
the headline workload.  `roofline` is for the dominant launch (gdn_prefill):
algorithmic FLOPs per launch / its average duration from HIP events on the
stream it runs on, against the published peak and against the peaks
measured in the same run (`measured_peaks`: the library's MFMA probe and a
1 GiB streaming copy); `hbm` is its secondary (bandwidth) ceiling.
`cpu_baseline` is the fp64 oracle timed on a bounded sample over a process
pool of the host's cores.
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
    taken on a different version of the kernel source (or of any other source
    whose hash it records)."""
    import hashlib
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip().lstrip("- ")] = v.strip().strip("`")
    shas = {k[len("sha256 "):]: v for k, v in fields.items() if k.startswith("sha256 ")}
    if source not in shas or "traffic_bytes_per_launch" not in fields:
        return None
    for name, want in shas.items():
        f = os.path.join(CSRC, name)
        if not os.path.exists(f) or hashlib.sha256(open(f, "rb").read()).hexdigest() != want:
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


def prefill_bytes_per_call(cfg, T, n_seqs, has_s0, state_bytes=4):
    """HBM bytes gdn_prefill must move at least once: q, k, v read and o
    written in the io dtype (bf16), g and beta (fp32), the initial state read
    (when given) and the final state written."""
    dk, dv, hq, hv = cfg["d_k"], cfg["d_v"], cfg["h_qk"], cfg["h_v"]
    per_tok = (2 * hq * dk + 2 * hv * dv) * 2 + 8 * hv
    st = n_seqs * hv * dv * dk * state_bytes
    return T * per_tok + st * (2 if has_s0 else 1)


_SHARED = {}  # oracle inputs handed to forked workers without pickling


def _pool_width(jobs):
    """Processes for an oracle pool: the host cores this process may use
    (capped at 16, the CPU share of one GPU on the box), at most one per job."""
    return max(1, min(len(os.sched_getaffinity(0)), 16, jobs))


def _oracle_prefill_job(job):
    from oracle import gdn_oracle as orc
    s = _SHARED
    t0, t1, heads = job
    orc.gdn_layer(s["x"][t0:t1], s["w"], s["g"][t0:t1], s["b"][t0:t1], s["hq"], s["d"], s["hv"], s["d"],
                  v_heads=heads)
    return (t1 - t0) * len(heads)


def cpu_baseline_prefill(inp, cfg, tokens):
    """The oracle (fp64 numpy, token by token) on a bounded sample of the
    workload: the first `tokens` tokens of every sequence (all of a shorter
    one), every V head, as (sequence, QK-head group) jobs over a process pool.
    The oracle is linear in tokens, so its rate is tokens / wall time."""
    import numpy as np
    import torch
    cu = [0, inp["T"]] if inp["cu_seqlens"] is None else inp["cu_seqlens"].tolist()
    grp = cfg["h_v"] // cfg["h_qk"]
    spans = [(cu[n], min(cu[n + 1], cu[n] + tokens)) for n in range(len(cu) - 1) if cu[n + 1] > cu[n]]
    jobs = [(a, b, list(range(qg * grp, (qg + 1) * grp))) for a, b in spans for qg in range(cfg["h_qk"])]
    sel = np.concatenate([np.arange(a, b) for a, b in spans])
    x = inp["x"][torch.from_numpy(sel)].double().numpy()
    # job token ranges are re-based onto the gathered sample
    base, off = [], 0
    for a, b in spans:
        base.append(off)
        off += b - a
    jobs = [(base[i // cfg["h_qk"]], base[i // cfg["h_qk"]] + (b - a), h) for i, (a, b, h) in enumerate(jobs)]
    _SHARED.update(x=x, w=inp["conv_weight"].double().numpy(), g=inp["g"].double().numpy()[sel],
                   b=inp["beta"].double().numpy()[sel], hq=cfg["h_qk"], d=cfg["d_k"], hv=cfg["h_v"])
    del x
    cores = _pool_width(len(jobs))
    ctx = mp.get_context("fork")
    t = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.map(_oracle_prefill_job, jobs, chunksize=1))
    dt = time.perf_counter() - t
    ntok = int(sum(b - a for a, b in spans))
    assert done == ntok * cfg["h_v"]
    return {"value": round(ntok / dt, 1), "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} tokens of each of {len(spans)} sequences ({ntok} of {inp['T']} tokens), "
                      f"all {cfg['h_v']} V heads, conv + recurrence, fp64 numpy, {len(jobs)} (sequence, QK group) "
                      f"jobs on {cores} processes; {dt:.1f} s"}


def flush_mall(scratch):
    """Overwrite a 1 GiB scratch buffer: evicts the 256 MB last-level cache."""
    scratch.fill_(1)


def run_prefill(name, steps, warmup, do_cpu, cpu_tokens, peaks, scratch):
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
    y = torch.empty_like(x)
    o = torch.empty((T, hv, d), dtype=x.dtype, device=dev)
    fs = torch.empty((N, hv, d, d), dtype=torch.float32, device=dev)
    q0, _, v0 = gdn.split_qkv(y, hq, d, hv, d)
    ws = torch.empty(max(1, gdn.prefill_workspace_size(q0, v0, N, cfg["chunk"])), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        gdn.conv1d(x, w, None, None, cu, "silu", out=y)
        q, k, v = gdn.split_qkv(y, hq, d, hv, d)
        if ev is not None:
            ev[1].record()
        gdn.prefill(q, k, v, g, beta, s0, cu, cfg["chunk"], 1.0, True, True, o=o, final_state=fs,
                    workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter()
    for i in range(steps):
        flush_mall(scratch)
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall) / steps * 1e3
    ms = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
    k_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    flops = prefill_flops_per_token(cfg) * T
    tflops = flops / (k_ms * 1e-3) / 1e12
    nbytes = prefill_bytes_per_call(cfg, T, N, s0 is not None)
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    res = {
        "tokens_per_s": T / (ms * 1e-3),
        "ms_per_step": ms,
        "wall_ms_per_step_with_flush": round(wall, 4),
        "prefill_kernel_ms": k_ms,
        "prefill_only_tokens_per_s": T / (k_ms * 1e-3),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(f"prefill_{name}_traffic.md", "prefill.hip"),
                     "kernel": "gdn_prefill",
                     "flops_per_launch": flops,
                     "frac_of_measured": round(tflops / peaks["mfma_bf16_tflops"], 4) if peaks else None},
        "hbm": {"bytes_per_launch": nbytes, "achieved": round(gbs, 1), "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4),
                "frac_of_measured": round(gbs / peaks["copy_gbs"], 4) if peaks else None},
        "config": {"workload": f"{name}: B={N} T={T} h_qk={hq} h_v={hv} d={d} "
                               f"chunk={cfg['chunk']} conv{cfg['width']}+SiLU, bf16 io, fp32 state",
                   "tokens": T, "n_seqs": N, "h_qk": hq, "h_v": hv, "d": d, "chunk": cfg["chunk"]},
    }
    if cu is not None:
        res["config"]["lengths"] = (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1]).tolist()
    if do_cpu:
        res["cpu_baseline"] = cpu_baseline_prefill(inp, cfg, cpu_tokens)
    del x, y, o, ws
    return res


def run_backward(name, steps, warmup, do_cpu, scratch):
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
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for i in range(steps):
        flush_mall(scratch)
        step(evs[i])
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[2]) for e in evs) / steps
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
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
    del ws, cws
    return res


def _oracle_decode_job(job):
    from oracle import gdn_oracle as orc
    s = _SHARED
    n0, n1 = job
    st, ct = s["S"][n0:n1].copy(), s["cs"][n0:n1].copy()
    for i in range(s["steps"]):
        _, st, ct = orc.decode_step(s["x"][i, n0:n1], s["w"], s["g"][i, n0:n1], s["b"][i, n0:n1], st, ct,
                                    s["hq"], s["d"], s["hv"], s["d"])
    return n1 - n0


def cpu_baseline_decode(inp, cfg, steps):
    """The oracle's decode over every sequence of the batch for `steps`
    steps, the sequences split over a process pool."""
    import numpy as np
    N = cfg["n_seqs"]
    cores = _pool_width(N)
    bounds = np.linspace(0, N, cores + 1).astype(int)
    jobs = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    _SHARED.update(S=inp["state"].double().numpy(), cs=inp["conv_state"].double().numpy(),
                   w=inp["conv_weight"].double().numpy(), x=inp["x"][:steps].double().numpy(),
                   g=inp["g"][:steps].double().numpy(), b=inp["beta"][:steps].double().numpy(), steps=steps,
                   hq=cfg["h_qk"], d=cfg["d_k"], hv=cfg["h_v"])
    ctx = mp.get_context("fork")
    t = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = sum(pool.map(_oracle_decode_job, jobs, chunksize=1))
    dt = (time.perf_counter() - t) / steps
    assert done == N
    return {"value": round(1.0 / dt, 3), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"all {N} sequences x {steps} steps, fp64 numpy, sequences split over {cores} processes"}


def run_decode(steps, warmup, do_cpu, state, peaks, cpu_steps=4):
    import torch
    import gdn_inputs
    import linear_attention_token_conv1d_amd as gdn

    inp = gdn_inputs.decode_inputs("qwen35_27b_decode", state=state)
    cfg = inp["cfg"]
    dev = torch.device("cuda:0")
    S = inp["state"].to(dev)
    cs = inp["conv_state"].to(dev)
    w = inp["conv_weight"].to(dev)
    xs, gs, bs = inp["x"].to(dev), inp["g"].to(dev), inp["beta"].to(dev)
    N, hq, hv, d = cfg["n_seqs"], cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    hd = torch.zeros(N, dtype=torch.int32, device=dev)  # conv-state ring heads
    o = torch.empty((N, hv, d), dtype=torch.bfloat16, device=dev)
    nsteps = xs.shape[0]
    # untimed: at least one full pass of the 64 steps (the clocks settle over
    # the first few dozen launches)
    for i in range(max(warmup, nsteps)):
        gdn.decode_step(xs[i % nsteps], gs[i % nsteps], bs[i % nsteps], S, hq, hv, d, conv_weight=w,
                        conv_state=cs, o=o, conv_head=hd)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(nsteps):
        gdn.decode_step(xs[i], gs[i], bs[i], S, hq, hv, d, conv_weight=w, conv_state=cs, o=o, conv_head=hd)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / nsteps
    nbytes = decode_bytes_per_step(cfg)
    gbs = nbytes / (ms * 1e-3) / 1e9
    st = "bf16" if state == "bf16" else "fp32"
    res = {"value": 1e3 / ms, "unit": "steps/s", "tokens_per_s": N * 1e3 / ms, "ms_per_step": ms,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": measured_traffic(f"decode_qwen35_27b_decode_{st}_traffic.md", "decode.hip"),
                        "kernel": f"decode_kernel<bf16,{st},128>", "bytes_per_launch": nbytes,
                        "frac_of_measured": round(gbs / peaks["copy_gbs"], 4) if peaks else None},
           "config": {"workload": f"qwen35_27b_decode: {N} sequences x 1 token, h_qk={hq} h_v={hv} d={d}, "
                                  f"{st} state, conv4+SiLU with a ring conv state, {nsteps} consecutive steps"}}
    del S, cs, xs
    if do_cpu:
        res["cpu_baseline"] = cpu_baseline_decode(inp, cfg, cpu_steps)
    return res


def torch_copy_gbs(nbytes=1 << 30, reps=5):
    """Best read + write rate of torch's own device-to-device copy of nbytes."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    best = 0.0
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best


def measure_peaks():
    """Ceilings measured on this machine: dense bf16 MFMA (the library's probe)
    and a 1 GiB streaming device copy (read + write bytes per second; the
    better of the library's copy probe and torch's copy)."""
    import linear_attention_token_conv1d_amd as gdn
    probe, tcopy = gdn.probe_copy(1 << 30), torch_copy_gbs(1 << 30)
    return {"mfma_bf16_tflops": round(gdn.probe_mfma(), 1), "copy_gbs": round(max(probe, tcopy), 1),
            "copy_probe_gbs": round(probe, 1), "torch_copy_gbs": round(tcopy, 1), "copy_bytes": 1 << 30}


EXTRA = {"qwen35_9b_prefill": "prefill_9b", "qwen35_27b_prefill": "prefill_27b", "qwen35_27b_varlen": "prefill_varlen"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen35_27b_varlen",
                    choices=["qwen35_9b_prefill", "qwen35_27b_prefill", "qwen35_27b_varlen"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="time only --workload (not the other two prefill workloads)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="oracle sample: this many tokens of every sequence")
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
    peaks = measure_peaks()
    print(f"# measured peaks {peaks}", file=sys.stderr, flush=True)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    do_cpu = not args.no_cpu_baseline
    pre = run_prefill(args.workload, args.steps, args.warmup, do_cpu, args.cpu_tokens, peaks, scratch)
    print(f"# {args.workload}: {pre['prefill_kernel_ms']:.4f} ms per gdn_prefill", file=sys.stderr, flush=True)
    line = {"metric": METRIC, "value": round(pre["tokens_per_s"], 1), "unit": "tokens/s/layer",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(pre["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": pre["config"], "roofline": pre["roofline"], "hbm": pre["hbm"],
            "measured_peaks": peaks,
            "prefill_kernel_ms": round(pre["prefill_kernel_ms"], 4),
            "prefill_only_tokens_per_s": round(pre["prefill_only_tokens_per_s"], 1),
            "wall_ms_per_step_with_flush": pre["wall_ms_per_step_with_flush"]}
    if "cpu_baseline" in pre:
        line["cpu_baseline"] = pre["cpu_baseline"]
    torch.cuda.empty_cache()
    if not args.no_extra_prefill:
        for name, key in EXTRA.items():
            if name == args.workload:
                continue
            r = run_prefill(name, args.steps, args.warmup, False, args.cpu_tokens, peaks, scratch)
            print(f"# {name}: {r['prefill_kernel_ms']:.4f} ms per gdn_prefill", file=sys.stderr, flush=True)
            line[key] = {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                         "prefill_kernel_ms": round(r["prefill_kernel_ms"], 4),
                         "prefill_only_tokens_per_s": round(r["prefill_only_tokens_per_s"], 1),
                         "roofline": r["roofline"], "hbm": r["hbm"], "config": r["config"]}
            torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = run_decode(args.steps, args.warmup, do_cpu, "bf16", peaks)
        torch.cuda.empty_cache()
        line["decode_fp32_state"] = run_decode(args.steps, args.warmup, do_cpu, "f32", peaks)
        torch.cuda.empty_cache()
    if not args.no_backward:
        line["backward"] = run_backward("qwen35_9b_prefill", args.steps, args.warmup, do_cpu, scratch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
