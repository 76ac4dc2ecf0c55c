"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (gdn_conv1d then gdn_prefill over the whole layer; gdn_decode_step on
the whole batch).  The GPU computes everything; the fp64 oracle recomputes a
sample it can afford -- whole V-head groups or whole sequences, over every
token -- and the two are compared element by element on that sample
(norm-wise relative error per tensor)."""
import time

import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn
from oracle import gdn_oracle as orc
from parity import TOL_BF16, TOL_F32, dev, np64, rel_err, rel_err_per, report

pytestmark = pytest.mark.gpu


def _run_layer(name, heads, **kw):
    t0 = time.time()
    inp = gdn_inputs.prefill_inputs(name, **kw)
    cfg = inp["cfg"]
    T, N, hq, hv, d = inp["T"], inp["n_seqs"], cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    print(f"[{name}] inputs T={T} N={N} ready in {time.time() - t0:.1f}s", flush=True)
    C = gdn_inputs.channels(cfg)
    cs = torch.zeros((N, C, cfg["width"] - 1), dtype=torch.bfloat16, device="cuda")
    cu = dev(inp["cu_seqlens"])
    o, S = gdn.gdn_layer(dev(inp["x"]), dev(inp["conv_weight"]), dev(inp["g"]), dev(inp["beta"]),
                         hq, d, hv, d, conv_state=cs, initial_state=dev(inp["initial_state"]),
                         cu_seqlens=cu, chunk=cfg["chunk"])
    torch.cuda.synchronize()
    o_s, S_s = o[:, heads].cpu(), S[:, heads].cpu()
    ch = orc.layer_channels(hq, d, hv, d, heads)
    cs_s = cs[:, torch.from_numpy(ch).cuda()].cpu()
    del o, S
    print(f"[{name}] GPU done; oracle on V heads {heads}", flush=True)
    t0 = time.time()
    chi = torch.from_numpy(ch)
    ro, rS, rcs = orc.gdn_layer(np64(inp["x"][:, chi]), np64(inp["conv_weight"][chi]), np64(inp["g"]),
                                np64(inp["beta"]), hq, d, hv, d, initial_state=np64(inp["initial_state"]),
                                cu_seqlens=None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy(),
                                v_heads=heads, x_is_selected=True)
    print(f"[{name}] oracle {time.time() - t0:.1f}s", flush=True)
    e = dict(o=rel_err(o_s, ro), state=rel_err(S_s, rS), conv_state=rel_err(cs_s, rcs),
             o_per_head=rel_err_per(o_s, ro, 1), state_per_head=rel_err_per(S_s, rS, 1))
    if inp["cu_seqlens"] is not None:  # each sequence on its own
        cu = inp["cu_seqlens"].numpy()
        e["o_per_seq"] = max(rel_err(o_s[cu[n]:cu[n + 1]], ro[cu[n]:cu[n + 1]])
                             for n in range(N) if cu[n + 1] > cu[n])
        e["state_per_seq"] = rel_err_per(S_s, rS, 0)
    report(f"[{name}] heads {heads}", **e)
    return e


def _ok(e):
    return all(v < TOL_BF16 for k, v in e.items() if k != "conv_state") and e["conv_state"] == 0.0


def test_qwen35_9b_layer_prefill():
    e = _run_layer("qwen35_9b_prefill", [0, 13, 31])
    assert _ok(e)


def test_qwen35_27b_grouped_prefill():
    # the first QK group whole, and heads of the last group (placement deals
    # QK groups round-robin over the XCDs)
    e = _run_layer("qwen35_27b_prefill", [0, 1, 2, 46, 47])
    assert _ok(e)


def test_qwen35_27b_varlen_prefill():
    # V heads of the first, middle and last QK groups, over all 8 sequences
    e = _run_layer("qwen35_27b_varlen", [0, 7, 24, 47])
    assert _ok(e)


def test_qwen35_27b_batched_decode_64_steps():
    inp = gdn_inputs.decode_inputs("qwen35_27b_decode")
    cfg = inp["cfg"]
    N, hq, hv, d = cfg["n_seqs"], cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    S, cs = dev(inp["state"]), dev(inp["conv_state"])
    w = dev(inp["conv_weight"])
    xs, gs, bs = dev(inp["x"]), dev(inp["g"]), dev(inp["beta"])
    # the conv state as a ring (head 0 at the start), as bench.py runs it
    hd = torch.zeros(N, dtype=torch.int32, device="cuda")
    outs = []
    for i in range(cfg["steps"]):
        outs.append(gdn.decode_step(xs[i], gs[i], bs[i], S, hq, hv, d, conv_weight=w, conv_state=cs,
                                    conv_head=hd))
    torch.cuda.synchronize()
    assert bool((hd == cfg["steps"] % (cfg["width"] - 1)).all())
    seqs = [0, 1, 37, 77, 128, 200, 254, 255]  # spread over the batch, the last included
    o_gpu = torch.stack(outs)[:, seqs].cpu()
    rS, rcs = np64(inp["state"][seqs]), np64(inp["conv_state"][seqs])
    dS = rS.copy()
    dcs = rcs.copy()
    ro, do = [], []
    wn = np64(inp["conv_weight"])
    for i in range(cfg["steps"]):
        xi, gi, bi = np64(inp["x"][i, seqs]), np64(inp["g"][i, seqs]), np64(inp["beta"][i, seqs])
        o_i, rS, rcs = orc.decode_step(xi, wn, gi, bi, rS, rcs, hq, d, hv, d)
        od_i, dS, dcs = orc.decode_step(xi, wn, gi, bi, dS, dcs, hq, d, hv, d, round_state_bf16=True)
        ro.append(o_i)
        do.append(od_i)
    cs_chrono = orc.ring_to_chronological(np64(cs[seqs]), hd[seqs].cpu().numpy())
    e = dict(o=rel_err(o_gpu, np.stack(ro)), state=rel_err(S[seqs].cpu(), rS),
             conv_state=rel_err(cs_chrono, rcs), o_per_seq=rel_err_per(o_gpu, np.stack(ro), 1),
             state_per_seq=rel_err_per(S[seqs].cpu(), rS, 0))
    diag = dict(o_vs_bf16_oracle=rel_err(o_gpu, np.stack(do)), state_vs_bf16_oracle=rel_err(S[seqs].cpu(), dS))
    report(f"[qwen35_27b_decode] seqs {seqs}", **e, **diag)
    assert _ok(e)


def test_tiny_fp32_layer_every_head():
    inp = gdn_inputs.prefill_inputs("tiny_fp32")
    o, S = gdn.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                       None, chunk=16)
    ro, rS = orc.gated_delta_rule(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["g"]),
                                  np64(inp["beta"]))
    assert rel_err(o, ro) < TOL_F32 and rel_err(S, rS) < TOL_F32
