"""GPU parity of the backward entry points (gdn_prefill_backward,
gdn_conv1d_backward and the two chained for a layer) against the fp64
oracle's backward.  The oracle's backward is pinned separately, by finite
differences and closed forms, in test_oracle_backward_pins.py.

Cases span several chunks with ragged tails, an empty and a one-token
sequence, chunk sizes 16/32/64, d 64/128, grouped heads, fp32 and bf16,
erase on and off, with and without the L2 norm; plus the 9B-shaped
workload at full size, checked on sampled heads."""
import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn
from oracle import gdn_oracle as orc
from parity import TOL_BF16, TOL_F32, dev, np64, rel_err, report

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}
NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]


def _rand(shape, dtype, std=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (std * torch.randn(shape, generator=g)).to(dtype)


def _gates(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    z1 = torch.randn((T, H), generator=g, dtype=torch.float64)
    z2 = torch.randn((T, H), generator=g, dtype=torch.float64)
    return torch.nn.functional.logsigmoid(z1).float(), torch.sigmoid(z2).float()


def _case(lens, h_qk, h_v, d, io, seed, s0=True, dsf=True):
    T = sum(lens)
    N = len(lens)
    q = _rand((T, h_qk, d), DT[io], seed=seed)
    k = _rand((T, h_qk, d), DT[io], seed=seed + 1)
    v = _rand((T, h_v, d), DT[io], seed=seed + 2)
    g, beta = _gates(T, h_v, seed + 3)
    S0 = _rand((N, h_v, d, d), torch.float32, 0.1, seed + 4) if s0 else None
    do = _rand((T, h_v, d), DT[io], seed=seed + 5)
    dSf = _rand((N, h_v, d, d), torch.float32, 0.3, seed + 6) if dsf else None
    cu = gdn_inputs.cu_from_lengths(lens) if N > 1 else None
    return q, k, v, g, beta, S0, do, dSf, cu


def _run_and_compare(lens, h_qk, h_v, d, io, chunk, erase=True, l2=True, s0=True, dsf=True, seed=0,
                     scale=1.0, tol=None):
    q, k, v, g, beta, S0, do, dSf, cu = _case(lens, h_qk, h_v, d, io, seed, s0, dsf)
    got = gdn.prefill_backward(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(do), dev(S0), dev(dSf), dev(cu),
                               chunk, scale, l2, erase)
    torch.cuda.synchronize()
    ref = orc.gated_delta_rule_backward(np64(q), np64(k), np64(v), np64(g), np64(beta), np64(do), np64(S0),
                                        np64(dSf), None if cu is None else cu.numpy(), scale, l2norm_qk=l2,
                                        erase=erase)
    errs = {n: rel_err(a, b) for n, a, b in zip(NAMES, got, ref)}
    report(f"prefill_backward[{io},d={d},C={chunk},erase={erase},l2={l2}]", **errs)
    tol = tol or (TOL_BF16 if io == "bf16" else TOL_F32)
    for n, e in errs.items():
        assert e < tol, (n, e)
    return got


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d,chunk", [(64, 16), (64, 64), (128, 32), (128, 64)])
@pytest.mark.parametrize("h_qk,h_v", [(2, 4), (3, 3)])
def test_prefill_backward_varlen_grouped(io, d, chunk, h_qk, h_v):
    """Two V heads per QK head (dq, dk summed over the group by the QK-head
    kernel) and one (the chunk-local kernel goes back through the L2 norm)."""
    _run_and_compare([70, 1, 0, 130, 33], h_qk, h_v, d, io, chunk, seed=10)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("h_qk,h_v", [(1, 3), (2, 2)])
def test_prefill_backward_erase_off(io, h_qk, h_v):
    _run_and_compare([150, 7], h_qk, h_v, 64, io, 64, erase=False, seed=20)


@pytest.mark.parametrize("io,d,chunk,T,h_qk,h_v,mb,opt", [
    ("bf16", 128, 64, 1000, 2, 4, 13, True),   # 4 windows of 256 tokens, the last ragged
    ("f32", 64, 32, 611, 2, 2, 4, True),       # fp32, chunk 32
    ("bf16", 64, 64, 777, 1, 3, 8, False),     # grouped heads, no initial state or final-state gradient
])
def test_prefill_backward_in_windows(monkeypatch, io, d, chunk, T, h_qk, h_v, mb, opt):
    """One sequence whose workspace passes the budget runs in windows: a
    forward pass for the window-start states, then each window's backward from
    the last to the first with the state gradient carried between them.  A
    small budget (GDN_BWD_BUDGET_MB) forces several windows here; the results
    must meet the same bar against the oracle as the whole-call backward."""
    monkeypatch.setenv("GDN_BWD_BUDGET_MB", str(mb))
    q = torch.empty((T, h_qk, d), dtype=DT[io])
    v = torch.empty((T, h_v, d), dtype=DT[io])
    monkeypatch.delenv("GDN_BWD_BUDGET_MB")
    full = gdn.prefill_backward_workspace_size(q, v, 1, chunk)
    monkeypatch.setenv("GDN_BWD_BUDGET_MB", str(mb))
    assert gdn.prefill_backward_workspace_size(q, v, 1, chunk) < full
    _run_and_compare([T], h_qk, h_v, d, io, chunk, s0=opt, dsf=opt, seed=90)


@pytest.mark.parametrize("io,d,chunk,lens,h_qk,h_v,mb,opt", [
    ("bf16", 128, 64, [520, 0, 333, 127], 2, 4, 13, True),   # the longest sequence also in windows
    ("f32", 64, 32, [300, 250, 150], 1, 3, 8, False),        # grouped heads, no initial state or final-state gradient
])
def test_prefill_backward_pack_one_sequence_at_a_time(monkeypatch, io, d, chunk, lens, h_qk, h_v, mb, opt):
    """A pack whose whole-call workspace passes the budget runs its sequences
    one after another (each in windows when long) in a workspace sized for one
    sequence of every token; the results meet the same bar against the
    oracle."""
    T = sum(lens)
    q = torch.empty((T, h_qk, d), dtype=DT[io])
    v = torch.empty((T, h_v, d), dtype=DT[io])
    full = gdn.prefill_backward_workspace_size(q, v, len(lens), chunk)
    monkeypatch.setenv("GDN_BWD_BUDGET_MB", str(mb))
    assert gdn.prefill_backward_workspace_size(q, v, len(lens), chunk) < full
    _run_and_compare(lens, h_qk, h_v, d, io, chunk, s0=opt, dsf=opt, seed=95)


def test_prefill_backward_pack_one_at_a_time_refused_under_stream_capture(monkeypatch):
    """The one-sequence-at-a-time pack reads the sequence offsets back, so
    under stream capture it returns an error before any launch (nothing is
    recorded); the same call then runs eagerly and meets the oracle bar."""
    monkeypatch.setenv("GDN_BWD_BUDGET_MB", "8")
    lens, h_qk, h_v, d, chunk = [300, 250, 150], 1, 3, 64, 32
    q, k, v, g, beta, S0, do, dSf, cu = _case(lens, h_qk, h_v, d, "f32", 96)
    qd, kd, vd, gd, bd, S0d, dod, dSfd, cud = (dev(t) for t in (q, k, v, g, beta, S0, do, dSf, cu))
    outs = dict(dq=torch.empty_like(qd), dk=torch.empty_like(kd), dv=torch.empty_like(vd), dg=torch.empty_like(gd),
                dbeta=torch.empty_like(bd), d_initial_state=torch.empty_like(S0d))
    ws = torch.empty(gdn.prefill_backward_workspace_size(qd, vd, len(lens), chunk), dtype=torch.uint8,
                     device=qd.device)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    refused = False
    with torch.cuda.graph(graph):
        try:
            gdn.prefill_backward(qd, kd, vd, gd, bd, dod, S0d, dSfd, cud, chunk, workspace=ws, **outs)
        except gdn.GdnError:
            refused = True
    assert refused
    got = gdn.prefill_backward(qd, kd, vd, gd, bd, dod, S0d, dSfd, cud, chunk, workspace=ws, **outs)
    torch.cuda.synchronize()
    ref = orc.gated_delta_rule_backward(np64(q), np64(k), np64(v), np64(g), np64(beta), np64(do), np64(S0),
                                        np64(dSf), cu.numpy(), 1.0)
    for n, a, b in zip(NAMES, got, ref):
        assert rel_err(a, b) < TOL_F32, n


def test_prefill_backward_without_l2_norm_and_scale():
    """Raw (unnormalised) small keys keep the recurrence bounded without the norm."""
    lens, h, d = [90], 2, 64
    q, k, v, g, beta, S0, do, dSf, cu = _case(lens, h, h, d, "f32", 30)
    k = k / 12.0
    q = q / 12.0
    got = gdn.prefill_backward(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(do), dev(S0), dev(dSf), None, 32,
                               0.5, False)
    torch.cuda.synchronize()
    ref = orc.gated_delta_rule_backward(np64(q), np64(k), np64(v), np64(g), np64(beta), np64(do), np64(S0),
                                        np64(dSf), None, 0.5, l2norm_qk=False)
    for n, a, b in zip(NAMES, got, ref):
        assert rel_err(a, b) < TOL_F32, n


def test_prefill_backward_null_optionals_and_single_tokens():
    """No initial state, no final-state gradient, d_initial_state still formed;
    sequences of one token and an empty one at the start and the end."""
    _run_and_compare([0, 1, 65, 1, 0], 2, 2, 128, "bf16", 64, s0=False, dsf=False, seed=40)


def test_prefill_backward_chunk_size_invariance():
    """The gradients do not depend on the chunk size beyond rounding."""
    args = _case([200, 45], 2, 4, 64, "f32", 50)
    q, k, v, g, beta, S0, do, dSf, cu = args
    outs = [gdn.prefill_backward(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(do), dev(S0), dev(dSf), dev(cu),
                                 c) for c in (16, 32, 64)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for n, a, b in zip(NAMES, outs[0], o):
            assert rel_err(a, np64(b)) < 1e-5, n


def test_prefill_backward_deterministic_and_writes_into_views():
    """Bitwise-identical repeats; dq, dk, dv written into column slices of one
    [T, C] gradient buffer leave the other columns untouched."""
    h_qk, h_v, d = 2, 4, 64
    q, k, v, g, beta, S0, do, dSf, cu = _case([100, 60], h_qk, h_v, d, "bf16", 60)
    T = q.shape[0]
    C = 2 * h_qk * d + h_v * d
    dy = torch.full((T, C + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = gdn.split_qkv(dy[:, :C], h_qk, d, h_v, d)
    r1 = gdn.prefill_backward(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(do), dev(S0), dev(dSf), dev(cu),
                              dq=dq, dk=dk, dv=dv)
    r2 = gdn.prefill_backward(dev(q), dev(k), dev(v), dev(g), dev(beta), dev(do), dev(S0), dev(dSf), dev(cu))
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    assert torch.equal(dy[:, C:], torch.full((T, 64), 7.0, dtype=torch.bfloat16, device="cuda"))


# ------------------------------------------------------------------- conv

@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("width,act", [(4, "silu"), (2, None), (3, "silu")])
def test_conv1d_backward_varlen_with_state(io, width, act):
    lens = [5, 1, 0, 2, 130, 3, 64, 70]
    T, C = sum(lens), 264
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((T, C), DT[io], seed=1)
    w = _rand((C, width), DT[io], 0.5, seed=2)
    bias = _rand((C,), DT[io], 0.1, seed=3)
    st = _rand((len(lens), C, width - 1), DT[io], seed=4)
    dy = _rand((T, C), DT[io], seed=5)
    dns = _rand((len(lens), C, width - 1), torch.float32, seed=6)
    dx, dw, db, dst = gdn.conv1d_backward(dev(x), dev(w), dev(dy), dev(bias), dev(st), dev(cu), act, dev(dns))
    torch.cuda.synchronize()
    ref = orc.causal_conv1d_backward(np64(x), np64(w), np64(dy), np64(bias), np64(st), cu.numpy(), act, np64(dns))
    errs = {n: rel_err(a, b) for n, a, b in zip(["dx", "dw", "db", "dstate"], (dx, dw, db, dst), ref)}
    report(f"conv1d_backward[{io},W={width},{act}]", **errs)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    for n, e in errs.items():
        assert e < tol, (n, e)


def test_conv1d_backward_no_state_no_bias_single_sequence():
    T, C = 300, 128
    x = _rand((T, C), torch.float32, seed=7)
    w = _rand((C, 4), torch.float32, 0.5, seed=8)
    dy = _rand((T, C), torch.float32, seed=9)
    dx, dw, db, dst = gdn.conv1d_backward(dev(x), dev(w), dev(dy))
    torch.cuda.synchronize()
    rdx, rdw, _, rdst = orc.causal_conv1d_backward(np64(x), np64(w), np64(dy))
    assert db is None
    assert rel_err(dx, rdx) < TOL_F32 and rel_err(dw, rdw) < TOL_F32 and rel_err(dst, rdst) < TOL_F32


# ------------------------------------------------------------------ layer

@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_layer_backward_matches_oracle(io):
    """conv -> SiLU -> split -> L2 norm -> recurrence, gradients of every input
    of the layer (x, conv weight, g, beta, initial state, conv state)."""
    lens = [120, 0, 77, 1]
    h_qk, h_v, d = 1, 2, 64
    T, N = sum(lens), len(lens)
    C = 2 * h_qk * d + h_v * d
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((T, C), DT[io], seed=70)
    w = _rand((C, 4), DT[io], 0.5, seed=71)
    cs = _rand((N, C, 3), DT[io], seed=72)
    g, beta = _gates(T, h_v, 73)
    S0 = _rand((N, h_v, d, d), torch.float32, 0.1, 74)
    do = _rand((T, h_v, d), DT[io], seed=75)
    dSf = _rand((N, h_v, d, d), torch.float32, 0.3, 76)
    dns = _rand((N, C, 3), torch.float32, seed=77)
    got = gdn.gdn_layer_backward(dev(x), dev(w), dev(g), dev(beta), h_qk, d, h_v, d, dev(do), None, dev(cs),
                                 dev(S0), dev(cu), 64, 1.0, True, True, dev(dSf), dev(dns))
    torch.cuda.synchronize()
    # oracle: forward conv, recurrence backward, the channel gradients stacked
    # as [q | k | v], then the conv backward
    cun = cu.numpy()
    y, _ = orc.causal_conv1d(np64(x), np64(w), None, np64(cs), cun)
    q, k, v = orc.split_qkv(y, h_qk, d, h_v, d)
    dq, dk, dv, dg, db, ds0 = orc.gated_delta_rule_backward(q, k, v, np64(g), np64(beta), np64(do), np64(S0),
                                                            np64(dSf), cun)
    dy = np.concatenate([dq.reshape(T, -1), dk.reshape(T, -1), dv.reshape(T, -1)], axis=1)
    dx, dw, _, dcs = orc.causal_conv1d_backward(np64(x), np64(w), dy, None, np64(cs), cun, "silu", np64(dns))
    names = ["dx", "dw", "dg", "dbeta", "dS0", "dconv_state"]
    vals = [got[0], got[1], got[3], got[4], got[5], got[6]]
    refs = [dx, dw, dg, db, ds0, dcs]
    errs = {n: rel_err(a, b) for n, a, b in zip(names, vals, refs)}
    report(f"layer_backward[{io}]", **errs)
    assert got[2] is None
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    for n, e in errs.items():
        assert e < tol, (n, e)


# ------------------------------------------------------ full size, sampled

def test_prefill_backward_9b_size_sampled_heads():
    """The 9B-shaped layer at full length (T = 8192, 32 + 32 heads, d = 128,
    chunk 64) through conv + split, then prefill_backward in one call; the
    oracle checks V heads 0 and 31 (with their QK heads: one V head per QK
    head here), which are independent of the others."""
    inp = gdn_inputs.prefill_inputs("qwen35_9b_prefill", seed=0)
    cfg = inp["cfg"]
    h_qk, h_v, d = cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    T = inp["T"]
    y = gdn.conv1d(dev(inp["x"]), dev(inp["conv_weight"]))
    q, k, v = gdn.split_qkv(y, h_qk, d, h_v, d)
    do = _rand((T, h_v, d), torch.bfloat16, seed=80)
    g, beta = dev(inp["g"]), dev(inp["beta"])
    got = gdn.prefill_backward(q, k, v, g, beta, dev(do))
    torch.cuda.synchronize()
    for h in (0, h_v - 1):
        hq = h // (h_v // h_qk)
        ref = orc.gated_delta_rule_backward(np64(q[:, hq:hq + 1]), np64(k[:, hq:hq + 1]), np64(v[:, h:h + 1]),
                                            np64(g[:, h:h + 1]), np64(beta[:, h:h + 1]), np64(do[:, h:h + 1]),
                                            segment=64)
        mine = [got[0][:, hq:hq + 1], got[1][:, hq:hq + 1], got[2][:, h:h + 1], got[3][:, h:h + 1],
                got[4][:, h:h + 1], got[5][:, h:h + 1]]
        errs = {n: rel_err(a, b) for n, a, b in zip(NAMES, mine, ref)}
        report(f"prefill_backward[9B, head {h}]", **errs)
        for n, e in errs.items():
            assert e < TOL_BF16, (h, n, e)


def test_prefill_backward_27b_size_sampled_group():
    """The 27B-shaped layer at full length (T = 65,536, 16 QK / 48 V heads,
    1,024 chunks, a non-zero initial state; the backward runs in windows under
    the default 4 GiB workspace budget) through conv + split,
    then prefill_backward with a final-state gradient; the oracle checks QK
    head groups 0 and 15 (V heads 0-2 and 45-47: the first and the last group,
    which the workgroup placement puts on different XCDs), whose gradients
    depend on no other head."""
    inp = gdn_inputs.prefill_inputs("qwen35_27b_prefill", seed=0)
    cfg = inp["cfg"]
    h_qk, h_v, d = cfg["h_qk"], cfg["h_v"], cfg["d_k"]
    T, grp = inp["T"], h_v // h_qk
    y = gdn.conv1d(dev(inp["x"]), dev(inp["conv_weight"]))
    q, k, v = gdn.split_qkv(y, h_qk, d, h_v, d)
    do = _rand((T, h_v, d), torch.bfloat16, seed=90)
    dsf = _rand((1, h_v, d, d), torch.float32, 0.3, seed=91)
    g, beta, s0 = dev(inp["g"]), dev(inp["beta"]), dev(inp["initial_state"])
    got = gdn.prefill_backward(q, k, v, g, beta, dev(do), s0, dev(dsf))
    torch.cuda.synchronize()
    for qg in (0, h_qk - 1):
        hs, qs = slice(qg * grp, (qg + 1) * grp), slice(qg, qg + 1)
        ref = orc.gated_delta_rule_backward(np64(q[:, qs]), np64(k[:, qs]), np64(v[:, hs]), np64(g[:, hs]),
                                            np64(beta[:, hs]), np64(do[:, hs]), np64(s0[:, hs]),
                                            np64(dsf[:, hs]), segment=64)
        mine = [got[0][:, qs], got[1][:, qs], got[2][:, hs], got[3][:, hs], got[4][:, hs], got[5][:, hs]]
        errs = {n: rel_err(a, b) for n, a, b in zip(NAMES, mine, ref)}
        report(f"prefill_backward[27B, group {qg}]", **errs)
        for n, e in errs.items():
            assert e < TOL_BF16, (qg, n, e)


@pytest.mark.parametrize("lens", [[0], [0, 0, 0]])
def test_backward_empty_inputs(lens):
    """No tokens at all: the state gradient passes straight through (or is
    zero without a final-state gradient), the conv weight gradient is zero and
    the conv-state gradient is the new-state gradient."""
    h_qk, h_v, d = 1, 2, 64
    N = len(lens)
    cu = gdn_inputs.cu_from_lengths(lens) if N > 1 else None
    q = torch.zeros((0, h_qk, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    v = torch.zeros((0, h_v, d), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((0, h_v), dtype=torch.float32, device="cuda")
    beta = torch.zeros_like(g)
    do = torch.zeros((0, h_v, d), dtype=torch.bfloat16, device="cuda")
    dsf = _rand((N, h_v, d, d), torch.float32, 0.3, seed=100).cuda()
    got = gdn.prefill_backward(q, k, v, g, beta, do, None, dsf, dev(cu))
    got0 = gdn.prefill_backward(q, k, v, g, beta, do, None, None, dev(cu))
    torch.cuda.synchronize()
    assert torch.equal(got[5], dsf)
    assert torch.count_nonzero(got0[5]).item() == 0
    C = 2 * h_qk * d + h_v * d
    x = torch.zeros((0, C), dtype=torch.bfloat16, device="cuda")
    w = _rand((C, 4), torch.bfloat16, 0.5, seed=101).cuda()
    dns = _rand((N, C, 3), torch.float32, seed=102).cuda()
    dx, dw, _, dst = gdn.conv1d_backward(x, w, torch.zeros_like(x), None, None, dev(cu), "silu", dns)
    torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.count_nonzero(dw).item() == 0
    assert torch.equal(dst, dns)
