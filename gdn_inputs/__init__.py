"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

Shared by the oracle-side and the HIP-side of every test and by the bench, so
that both sides see bit-identical inputs.  It holds none of the mixer's own
arithmetic: only random draws, their documented distributions, the rounding
of each draw to the io dtype, and the packing of sequences.

Every draw comes from one numpy Generator(PCG64(seed)) in the order listed in
each function.  Draws are made in float32 (float64 for the gate
pre-activations), then rounded to the io dtype with round-to-nearest-even
(torch's CPU cast).  Returned tensors are torch CPU tensors holding exactly
the values the kernels receive.

Workload shapes (the 9B and 27B shapes follow the layer configuration the
pages quote: "Inside Qwen3.5", config note -- Gated DeltaNet with 16 QK and
48 V heads of width 128, conv kernel 4; "Qwen3.5-9B vs Qwen3-8B measured",
section 1 -- 32 heads of 128 x 128 state per layer in the 9B).
"""
from __future__ import annotations

import math

import numpy as np
import torch

ROW_BLOCK = 4096  # tokens per draw block for the large x tensors


def _dt(name):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


CONFIGS = {
    # tiny fp32 layer: no conv, raw q/k/v normalised by the kernel
    "tiny_fp32": dict(kind="prefill", n_seqs=1, T=256, h_qk=4, h_v=4, d_k=64, d_v=64, chunk=16,
                      io="f32", conv=False, state_std=0.0),
    # 9B-shaped layer prefill
    "qwen35_9b_prefill": dict(kind="prefill", n_seqs=1, T=8192, h_qk=32, h_v=32, d_k=128, d_v=128,
                              chunk=64, io="bf16", conv=True, width=4, conv_std=0.5, state_std=0.0),
    # 27B-shaped prefill with grouped heads and a random initial state
    "qwen35_27b_prefill": dict(kind="prefill", n_seqs=1, T=65536, h_qk=16, h_v=48, d_k=128,
                               d_v=128, chunk=64, io="bf16", conv=True, width=4, conv_std=0.5,
                               state_std=0.1),
    # batched decode, 27B shape, bf16 state
    "qwen35_27b_decode": dict(kind="decode", n_seqs=256, steps=64, h_qk=16, h_v=48, d_k=128,
                              d_v=128, io="bf16", state="bf16", width=4, conv_std=0.5,
                              state_std=0.1),
    # varlen packed prefill, 27B shape
    "qwen35_27b_varlen": dict(kind="prefill", n_seqs=8, T=262144, len_min=4096, len_max=65536,
                              h_qk=16, h_v=48, d_k=128, d_v=128, chunk=64, io="bf16", conv=True,
                              width=4, conv_std=0.5, state_std=0.0),
}


def channels(cfg):
    """Conv channels of the concatenated [q | k | v]."""
    return 2 * cfg["h_qk"] * cfg["d_k"] + cfg["h_v"] * cfg["d_v"]


def _round(a, io):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_dt(io))


def _normal_rows(rng, rows, cols, io):
    """[rows, cols] N(0,1) in io dtype, drawn in blocks of ROW_BLOCK rows."""
    out = torch.empty((rows, cols), dtype=_dt(io))
    for r0 in range(0, rows, ROW_BLOCK):
        r1 = min(rows, r0 + ROW_BLOCK)
        out[r0:r1] = _round(rng.standard_normal((r1 - r0, cols), dtype=np.float32), io)
    return out


def _gates(rng, shape):
    """g = logsigmoid(z1), beta = sigmoid(z2) with z ~ N(0,1) (float64, stored fp32)."""
    z1 = rng.standard_normal(shape)
    g = -np.logaddexp(0.0, -z1)
    z2 = rng.standard_normal(shape)
    beta = 1.0 / (1.0 + np.exp(-z2))
    return (torch.from_numpy(g.astype(np.float32)), torch.from_numpy(beta.astype(np.float32)))


def varlen_lengths(n, total, lo, hi, rng):
    """Sequence lengths log-uniform in [lo, hi], rescaled to sum to `total`.

    Draw u_i ~ U(ln lo, ln hi), L_i = e^{u_i}; rescale to the total; clip to
    [lo, hi] and rescale the unclipped ones, until stable; round down and add
    the remainder to the longest unclipped length."""
    assert n * lo <= total <= n * hi
    L = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    clipped = np.zeros(n, dtype=bool)
    for _ in range(100):
        free = ~clipped
        rest = total - L[clipped].sum()
        L[free] *= rest / L[free].sum()
        newly = free & ((L < lo) | (L > hi))
        if not newly.any():
            break
        L = np.clip(L, lo, hi)
        clipped |= newly
    Li = np.floor(L).astype(np.int64)
    free_idx = np.where(~clipped)[0] if (~clipped).any() else np.arange(n)
    Li[free_idx[np.argmax(Li[free_idx])]] += total - Li.sum()
    assert Li.sum() == total and (Li >= lo).all() and (Li <= hi).all()
    return Li


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return torch.from_numpy(cu)


def prefill_inputs(name="qwen35_9b_prefill", seed=0, T=None, lengths=None, **over):
    """Inputs of one prefill workload.

    Draw order: [lengths (varlen only)], then x [T, C] (or q, k, v without a
    conv), conv weight [C, W] (std conv_std), g-preactivation [T, H_v],
    beta-preactivation [T, H_v], initial state [N, H_v, d_v, d_k] (std
    state_std, fp32) when state_std > 0.

    T / lengths override the workload's length (same distributions, fewer
    tokens); `over` overrides any config field (e.g. heads) for small cases.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    rng = np.random.default_rng(seed)
    if lengths is None and "len_min" in cfg and T is None:
        lengths = varlen_lengths(cfg["n_seqs"], cfg["T"], cfg["len_min"], cfg["len_max"], rng)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = cu_from_lengths(lengths)
    else:
        T = cfg["T"] if T is None else int(T)
        cu = None
    N = 1 if cu is None else len(lengths)
    io = cfg["io"]
    out = dict(cfg=cfg, T=T, n_seqs=N, cu_seqlens=cu)
    if cfg["conv"]:
        C = channels(cfg)
        out["x"] = _normal_rows(rng, T, C, io)
        out["conv_weight"] = _round(cfg["conv_std"] * rng.standard_normal((C, cfg["width"]),
                                                                          dtype=np.float32), io)
    else:
        for key, h, d in (("q", cfg["h_qk"], cfg["d_k"]), ("k", cfg["h_qk"], cfg["d_k"]),
                          ("v", cfg["h_v"], cfg["d_v"])):
            out[key] = _normal_rows(rng, T, h * d, io).reshape(T, h, d)
    out["g"], out["beta"] = _gates(rng, (T, cfg["h_v"]))
    if cfg["state_std"] > 0:
        s = rng.standard_normal((N, cfg["h_v"], cfg["d_v"], cfg["d_k"]), dtype=np.float32)
        out["initial_state"] = torch.from_numpy(cfg["state_std"] * s)
    else:
        out["initial_state"] = None
    return out


def decode_inputs(name="qwen35_27b_decode", seed=0, n_seqs=None, steps=None, **over):
    """Inputs of the batched decode workload.

    Draw order: state [N, H_v, d_v, d_k] (std state_std, rounded to the state
    dtype), conv state [N, C, W-1] N(0,1) in io dtype, conv weight [C, W]
    (std conv_std), then per step: x [N, C] N(0,1), g-preactivation [N, H_v],
    beta-preactivation [N, H_v].
    """
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    if n_seqs is not None:
        cfg["n_seqs"] = n_seqs
    if steps is not None:
        cfg["steps"] = steps
    rng = np.random.default_rng(seed)
    N, Hv, dv, dk = cfg["n_seqs"], cfg["h_v"], cfg["d_v"], cfg["d_k"]
    C, W, io = channels(cfg), cfg["width"], cfg["io"]
    state = torch.empty((N, Hv, dv, dk), dtype=_dt(cfg["state"]))
    for n in range(N):
        state[n] = _round(cfg["state_std"] * rng.standard_normal((Hv, dv, dk), dtype=np.float32),
                          cfg["state"])
    conv_state = _normal_rows(rng, N, C * (W - 1), io).reshape(N, C, W - 1)
    conv_weight = _round(cfg["conv_std"] * rng.standard_normal((C, W), dtype=np.float32), io)
    xs, gs, bs = [], [], []
    for _ in range(cfg["steps"]):
        xs.append(_normal_rows(rng, N, C, io))
        g, b = _gates(rng, (N, Hv))
        gs.append(g)
        bs.append(b)
    return dict(cfg=cfg, state=state, conv_state=conv_state, conv_weight=conv_weight,
                x=torch.stack(xs), g=torch.stack(gs), beta=torch.stack(bs))
