"""GPU parity of every entry point against the fp64 oracle on small cases that
span several chunks/tiles, ragged tails and the degenerate cases: empty and
length-1..3 sequences, partial chunks, chunk sizes 16/32/64, d 64/128,
grouped heads, fp32 and bf16, with and without conv/L2 norm."""
import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn
from oracle import gdn_oracle as orc
from parity import TOL_BF16, TOL_F32, dev, np64, rel_err, report

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rand(shape, dtype, std=1.0, seed=0):
    g = torch.Generator().manual_seed(seed)
    return (std * torch.randn(shape, generator=g)).to(dtype)


def _gates(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    z1, z2 = torch.randn((T, H), generator=g, dtype=torch.float64), torch.randn((T, H), generator=g, dtype=torch.float64)
    return (torch.nn.functional.logsigmoid(z1).float(), torch.sigmoid(z2).float())


# ------------------------------------------------------------------ conv1d

@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("width", [4, 2])
def test_conv1d_varlen_with_state(io, width):
    lens = [5, 1, 0, 2, 130, 3, 64, 200]
    T, C = sum(lens), 520
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((T, C), DT[io], seed=1)
    w = _rand((C, width), DT[io], 0.5, seed=2)
    bias = _rand((C,), DT[io], 0.1, seed=3)
    st = _rand((len(lens), C, width - 1), DT[io], seed=4)
    st_d = dev(st.clone())
    y = gdn.conv1d(dev(x), dev(w), dev(bias), st_d, dev(cu))
    ry, rst = orc.causal_conv1d(np64(x), np64(w), np64(bias), np64(st), cu.numpy())
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    e_y, e_s = rel_err(y, ry), rel_err(st_d, rst)
    report(f"conv1d[{io},W={width}]", y=e_y, state=e_s)
    assert e_y < (4e-3 if io == "bf16" else 1e-6) and e_s == 0.0
    # without a state: zero history, nothing written
    y0 = gdn.conv1d(dev(x), dev(w), None, None, dev(cu))
    ry0, _ = orc.causal_conv1d(np64(x), np64(w), None, None, cu.numpy())
    assert rel_err(y0, ry0) < tol


def test_conv1d_single_sequence_no_activation():
    T, C = 77, 64
    x = _rand((T, C), torch.bfloat16, seed=5)
    w = _rand((C, 4), torch.bfloat16, 0.5, seed=6)
    y = gdn.conv1d(dev(x), dev(w), activation=None)
    ry, _ = orc.causal_conv1d(np64(x), np64(w), activation=None)
    assert rel_err(y, ry) < 4e-3


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("io,state_dt,d", [("bf16", "bf16", 128), ("bf16", "f32", 128),
                                           ("f32", "f32", 64), ("f32", "f32", 128),
                                           ("bf16", "bf16", 64)])
def test_decode_step_matches_oracle(io, state_dt, d):
    N, hq, hv = 5, 2, 6
    C = 2 * hq * d + hv * d
    x = _rand((N, C), DT[io], seed=7)
    w = _rand((C, 4), DT[io], 0.5, seed=8)
    cs = _rand((N, C, 3), DT[io], seed=9)
    S = _rand((N, hv, d, d), DT[state_dt], 0.1, seed=10)
    g, b = _gates(N, hv, 11)
    S_d, cs_d = dev(S.clone()), dev(cs.clone())
    o = gdn.decode_step(dev(x), dev(g), dev(b), S_d, hq, hv, d, conv_weight=dev(w), conv_state=cs_d)
    ro, rS, rcs = orc.decode_step(np64(x), np64(w), np64(g), np64(b), np64(S), np64(cs), hq, d, hv, d)
    tol = TOL_BF16 if "bf16" in (io, state_dt) else TOL_F32
    e = dict(o=rel_err(o, ro), state=rel_err(S_d, rS), conv_state=rel_err(cs_d, rcs))
    report(f"decode[{io},{state_dt},d={d}]", **e)
    assert e["o"] < tol and e["state"] < tol and e["conv_state"] == 0.0


@pytest.mark.parametrize("io,state_dt,d", [("bf16", "bf16", 128), ("f32", "f32", 64)])
def test_decode_step_erase_off(io, state_dt, d):
    """The erase-off variant (delta_i = beta v_i) against the oracle's additive
    recurrence, with the conv step."""
    N, hq, hv = 4, 2, 6
    C = 2 * hq * d + hv * d
    x = _rand((N, C), DT[io], seed=17)
    w = _rand((C, 4), DT[io], 0.5, seed=18)
    cs = _rand((N, C, 3), DT[io], seed=19)
    S = _rand((N, hv, d, d), DT[state_dt], 0.1, seed=20)
    g, b = _gates(N, hv, 21)
    S_d, cs_d = dev(S.clone()), dev(cs.clone())
    o = gdn.decode_step(dev(x), dev(g), dev(b), S_d, hq, hv, d, conv_weight=dev(w), conv_state=cs_d,
                        erase=False)
    ro, rS, rcs = orc.decode_step(np64(x), np64(w), np64(g), np64(b), np64(S), np64(cs), hq, d, hv, d,
                                  erase=False)
    tol = TOL_BF16 if "bf16" in (io, state_dt) else TOL_F32
    e = dict(o=rel_err(o, ro), state=rel_err(S_d, rS), conv_state=rel_err(cs_d, rcs))
    report(f"decode_erase_off[{io},{state_dt},d={d}]", **e)
    assert e["o"] < tol and e["state"] < tol and e["conv_state"] == 0.0


def test_decode_step_without_conv_64_steps():
    """No conv (x already holds q|k|v), 64 steps, fp32 io/state, 1e-4."""
    N, hq, hv, d = 3, 1, 2, 64
    C = 2 * hq * d + hv * d
    S = _rand((N, hv, d, d), torch.float32, 0.1, seed=12)
    S_d = dev(S.clone())
    rS = np64(S)
    for step in range(64):
        x = _rand((N, C), torch.float32, seed=100 + step)
        g, b = _gates(N, hv, 200 + step)
        o = gdn.decode_step(dev(x), dev(g), dev(b), S_d, hq, hv, d)
        ro, rS, _ = orc.decode_step(np64(x), None, np64(g), np64(b), rS, None, hq, d, hv, d)
        assert rel_err(o, ro) < TOL_F32
    assert rel_err(S_d, rS) < TOL_F32


# ------------------------------------------------------------------ prefill

def _prefill_case(T, hq, hv, d, io, seed, lens=None, s0=True):
    q = _rand((T, hq, d), DT[io], seed=seed)
    k = _rand((T, hq, d), DT[io], seed=seed + 1)
    v = _rand((T, hv, d), DT[io], seed=seed + 2)
    g, b = _gates(T, hv, seed + 3)
    N = 1 if lens is None else len(lens)
    S0 = _rand((N, hv, d, d), torch.float32, 0.1, seed=seed + 4) if s0 else None
    return q, k, v, g, b, S0


@pytest.mark.parametrize("io,d,chunk", [("bf16", 128, 64), ("bf16", 128, 32), ("bf16", 128, 16),
                                        ("bf16", 64, 64), ("f32", 64, 16), ("f32", 64, 32),
                                        ("f32", 128, 32)])
def test_prefill_ragged(io, d, chunk):
    T, hq, hv = 201, 2, 6
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, io, 20)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), chunk=chunk)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0))
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill[{io},d={d},C={chunk}]", **e)
    assert e["o"] < tol and e["state"] < tol


@pytest.mark.parametrize("T,hq,hv,d,chunk,s0,fin", [
    (2500, 2, 4, 128, 64, True, True),   # ragged last chunk, grouped heads
    (2048, 1, 1, 128, 64, False, True),  # whole chunks, one head, zero initial state
    (2113, 2, 2, 64, 64, True, True),    # d = 64: one 64-column block per head
    (1100, 2, 2, 128, 32, True, True),   # chunk 32
    (600, 1, 3, 128, 16, True, False),   # chunk 16, no final state asked for
    (2100, 8, 24, 128, 64, True, True),  # 32-column split with the second segment in two waves
    (2048, 8, 40, 128, 64, True, True),  # 64-column split
])
def test_prefill_one_long_sequence_split(T, hq, hv, d, chunk, s0, fin):
    """One sequence of 32+ chunks whose heads leave most CUs idle.  At chunk
    16 the scan runs the two halves side by side (the second from a zero
    state and as its own transition) and joins them; at chunks 32 and 64 the
    fused kernel runs one chain per column block over every chunk.  Outputs
    and final state must match the token-by-token oracle either way."""
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, "bf16", 90, s0=s0)
    if chunk == 16:
        # the split is in use: its workspace holds the extra states and outputs
        assert gdn.prefill_workspace_size(dev(q), dev(v), 1, chunk) > gdn.prefill_workspace_size(dev(q), dev(v), 2, chunk)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0) if s0 else None, chunk=chunk,
                       output_final_state=fin)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0) if s0 else None)
    e = dict(o=rel_err(o, ro))
    if fin:
        e["state"] = rel_err(S, rS)
    else:
        assert S is None
    report(f"prefill_split[T={T},h={hq}/{hv},d={d},C={chunk}]", **e)
    assert all(x < TOL_BF16 for x in e.values())


@pytest.mark.parametrize("io,d,chunk,T,lens", [
    ("bf16", 128, 64, 201, None),          # ragged tail, grouped heads
    ("f32", 64, 16, 150, None),            # fp32 path
    ("bf16", 64, 32, None, [40, 0, 130, 7]),  # varlen pack with an empty sequence
    ("bf16", 128, 64, 2500, None),         # one long sequence: split scan
])
def test_prefill_erase_off(io, d, chunk, T, lens):
    """The erase-off variant S_t = a_t S_{t-1} + b_t v_t k_t^T (same chunked
    path with A = 0, U = diag(beta) V) against the oracle's additive recurrence."""
    hq, hv = 2, 4
    if lens is not None:
        T = sum(lens)
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, io, 110, lens)
    cu = None if lens is None else gdn_inputs.cu_from_lengths(lens)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=chunk,
                       erase=False)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0),
                                  cu_seqlens=None if cu is None else cu.numpy(), erase=False)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill_erase_off[{io},d={d},C={chunk},T={T}]", **e)
    assert e["o"] < tol and e["state"] < tol


@pytest.mark.parametrize("io,d,chunk,K,lens", [
    ("bf16", 128, 64, 1, [200, 0, 300, 64, 65]),  # every chunk; empty and exact-chunk sequences
    ("f32", 64, 16, 3, [250]),                     # fp32 scan, every third chunk
    ("bf16", 128, 64, 2, [2500]),                  # one long sequence: the split is off when emitting
])
def test_prefill_chunk_state_emission(io, d, chunk, K, lens):
    """emit_every = K: the state after every K-th whole chunk that ends inside
    its sequence equals the oracle's final state over that prefix."""
    hq, hv = 2, 4
    T = sum(lens)
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, io, 120, lens)
    cu = gdn_inputs.cu_from_lengths(lens)
    o, S, E = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=chunk,
                          emit_every=K)
    rows = gdn.chunk_state_rows(lens, chunk, K)
    assert rows == sum((L - 1) // (K * chunk) for L in lens if L > 0)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0), cu_seqlens=cu.numpy())
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    assert rel_err(o, ro) < tol and rel_err(S, rS) < tol
    r, worst = 0, 0.0
    for n, L in enumerate(lens):
        s0 = int(cu[n])
        for j in range(1, (L - 1) // (K * chunk) + 1 if L > 0 else 1):
            e = s0 + j * K * chunk
            _, rSj = orc.gated_delta_rule(np64(q[s0:e]), np64(k[s0:e]), np64(v[s0:e]), np64(g[s0:e]),
                                          np64(b[s0:e]), np64(S0[n:n + 1]))
            worst = max(worst, rel_err(E[r:r + 1], rSj))
            r += 1
    assert r == rows
    report(f"chunk_states[{io},d={d},C={chunk},K={K}]", states=worst)
    assert worst < tol


@pytest.mark.parametrize("lens,slots,pool", [([70, 130, 5], [2, 0, 3], 4), ([2500], [3], 4)])
def test_prefill_state_slots(lens, slots, pool):
    """state_idx: sequence n starts from initial pool slot state_idx[n] and
    writes final pool slot state_idx[n]; other slots are left alone.  The
    single long sequence takes the split scan."""
    hq, hv, d = 2, 4, 128
    T = sum(lens)
    q, k, v, g, b, _ = _prefill_case(T, hq, hv, d, "bf16", 130, lens)
    P0 = _rand((pool, hv, d, d), torch.float32, 0.1, seed=131)
    cu = gdn_inputs.cu_from_lengths(lens)
    idx = torch.tensor(slots, dtype=torch.int32)
    fin = torch.full((pool, hv, d, d), 7.0, device="cuda")
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(P0), cu_seqlens=dev(cu), chunk=64,
                       final_state=fin, state_idx=dev(idx))
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(P0[idx.long()]),
                                  cu_seqlens=cu.numpy())
    e = dict(o=rel_err(o, ro), state=rel_err(fin[idx.long()], rS))
    report(f"state_slots[{lens}]", **e)
    assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16
    untouched = [i for i in range(pool) if i not in slots]
    assert bool((fin[untouched] == 7.0).all())


def test_decode_step_state_slots():
    """state_idx: the state and conv-state pools are addressed by slot; x, g,
    beta and o by sequence; slots no sequence names are left alone."""
    N, hq, hv, d, pool = 3, 2, 6, 128, 5
    C = 2 * hq * d + hv * d
    slots = [4, 1, 2]
    x = _rand((N, C), torch.bfloat16, seed=140)
    w = _rand((C, 4), torch.bfloat16, 0.5, seed=141)
    cs = _rand((pool, C, 3), torch.bfloat16, seed=142)
    S = _rand((pool, hv, d, d), torch.bfloat16, 0.1, seed=143)
    g, b = _gates(N, hv, 144)
    idx = torch.tensor(slots, dtype=torch.long)
    S_d, cs_d = dev(S.clone()), dev(cs.clone())
    o = gdn.decode_step(dev(x), dev(g), dev(b), S_d, hq, hv, d, conv_weight=dev(w), conv_state=cs_d,
                        state_idx=dev(idx.int()))
    ro, rS, rcs = orc.decode_step(np64(x), np64(w), np64(g), np64(b), np64(S[idx]), np64(cs[idx]), hq, d, hv, d)
    e = dict(o=rel_err(o, ro), state=rel_err(S_d[idx.cuda()], rS), conv_state=rel_err(cs_d[idx.cuda()], rcs))
    report("decode_state_slots", **e)
    assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16 and e["conv_state"] == 0.0
    for i in (0, 3):
        assert torch.equal(S_d[i].cpu(), S[i]) and torch.equal(cs_d[i].cpu(), cs[i])


def test_prefill_tiny_fp32_config():
    """The tiny fp32 layer: T=256, 4 heads, d=64, chunk 16, zero initial state."""
    inp = gdn_inputs.prefill_inputs("tiny_fp32")
    o, S = gdn.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]), dev(inp["beta"]),
                       None, chunk=16)
    ro, rS = orc.gated_delta_rule(np64(inp["q"]), np64(inp["k"]), np64(inp["v"]), np64(inp["g"]),
                                  np64(inp["beta"]))
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report("prefill[tiny_fp32]", **e)
    assert e["o"] < TOL_F32 and e["state"] < TOL_F32


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_prefill_varlen_degenerate_lengths(io):
    lens = [1, 2, 3, 0, 64, 65, 130, 17, 0]
    T, hq, hv, d = sum(lens), 1, 3, 64
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, io, 30, lens)
    cu = gdn_inputs.cu_from_lengths(lens)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu),
                       chunk=64 if io == "bf16" else 32)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0),
                                  cu_seqlens=cu.numpy())
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill_varlen[{io}]", **e)
    assert e["o"] < tol and e["state"] < tol
    # empty sequences pass their initial state through unchanged
    assert torch.equal(S[3].cpu(), S0[3]) and torch.equal(S[8].cpu(), S0[8])


def test_prefill_no_l2norm_and_scale():
    T, hq, hv, d = 100, 2, 2, 64
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, "f32", 40)
    k = torch.nn.functional.normalize(k, dim=-1)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), chunk=32, scale=0.25,
                       l2norm=False)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0), scale=0.25,
                                  l2norm_qk=False)
    assert rel_err(o, ro) < TOL_F32 and rel_err(S, rS) < TOL_F32


def test_prefill_chunk_size_invariance_and_determinism():
    T, hq, hv, d = 300, 2, 4, 128
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, "f32", 50)
    args = [dev(t) for t in (q, k, v, g, b, S0)]
    outs = [gdn.prefill(*args, chunk=c) for c in (16, 32)]
    assert rel_err(outs[0][0], np64(outs[1][0])) < 1e-5
    assert rel_err(outs[0][1], np64(outs[1][1])) < 1e-5
    again = gdn.prefill(*args, chunk=16)
    assert torch.equal(again[0], outs[0][0]) and torch.equal(again[1], outs[0][1])


def test_split_prefill_and_decode_continuation():
    """prefill(T1) then prefill(T2) == prefill(T1+T2); prefill(T) then one
    decode step (fp32 state, no conv) == prefill(T+1) -- all on the GPU."""
    T1, T2, hq, hv, d = 130, 71, 2, 4, 64
    T = T1 + T2
    q, k, v, g, b, S0 = _prefill_case(T + 1, hq, hv, d, "f32", 60)
    D = [dev(t) for t in (q, k, v, g, b)]
    S0d = dev(S0)
    o, S = gdn.prefill(*[t[:T] for t in D], S0d, chunk=32)
    oa, Sa = gdn.prefill(*[t[:T1] for t in D], S0d, chunk=32)
    ob, Sb = gdn.prefill(*[t[T1:T] for t in D], Sa, chunk=32)
    assert rel_err(torch.cat([oa, ob]), np64(o)) < 1e-5 and rel_err(Sb, np64(S)) < 1e-5
    o1, S1 = gdn.prefill(*D, S0d, chunk=32)
    x = torch.cat([D[0][T].reshape(1, -1), D[1][T].reshape(1, -1), D[2][T].reshape(1, -1)], dim=1)
    Sd = S.clone()
    od = gdn.decode_step(x.contiguous(), D[3][T:].contiguous(), D[4][T:].contiguous(), Sd, hq, hv, d)
    assert rel_err(od[0], np64(o1[T])) < 1e-5 and rel_err(Sd, np64(S1)) < 1e-5


def test_prefill_in_place_state_and_strided_inputs():
    """final_state may alias initial_state; q/k/v may be column slices of the
    conv output (token stride > heads)."""
    T, hq, hv, d = 150, 1, 3, 128
    C = 2 * hq * d + hv * d
    y = _rand((T, C), torch.bfloat16, seed=70)
    g, b = _gates(T, hv, 71)
    S0 = _rand((1, hv, d, d), torch.float32, 0.1, seed=72)
    yd = dev(y)
    q, k, v = gdn.split_qkv(yd, hq, d, hv, d)
    Sd = dev(S0.clone())
    o, S = gdn.prefill(q, k, v, dev(g), dev(b), Sd, final_state=Sd, chunk=64)
    assert S.data_ptr() == Sd.data_ptr()
    rq, rk, rv = orc.split_qkv(np64(y), hq, d, hv, d)
    ro, rS = orc.gated_delta_rule(rq, rk, rv, np64(g), np64(b), np64(S0))
    assert rel_err(o, ro) < TOL_BF16 and rel_err(Sd, rS) < TOL_BF16


def test_layer_conv_then_prefill():
    lens = [70, 1, 5, 129]
    T, hq, hv, d = sum(lens), 2, 6, 128
    C = 2 * hq * d + hv * d
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((T, C), torch.bfloat16, seed=80)
    w = _rand((C, 4), torch.bfloat16, 0.5, seed=81)
    g, b = _gates(T, hv, 82)
    cs = _rand((len(lens), C, 3), torch.bfloat16, seed=83)
    cs_d = dev(cs.clone())
    o, S = gdn.gdn_layer(dev(x), dev(w), dev(g), dev(b), hq, d, hv, d, conv_state=cs_d, cu_seqlens=dev(cu))
    ro, rS, rcs = orc.gdn_layer(np64(x), np64(w), np64(g), np64(b), hq, d, hv, d, conv_state=np64(cs),
                                cu_seqlens=cu.numpy())
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS), conv_state=rel_err(cs_d, rcs))
    report("layer[bf16]", **e)
    assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16 and e["conv_state"] == 0.0


@pytest.mark.parametrize("d,chunk", [(128, 64), (128, 32), (64, 64)])
def test_prefill_many_heads_wider_blocks(d, chunk):
    """Enough (sequence, V head) units that the fused kernel takes 32-column
    workgroups instead of 16-column ones: 9 sequences (an empty one, one
    token, exact and ragged chunks) x 8 V heads over 2 QK heads."""
    lens = [130, 0, 1, 64, 200, 65, 33, 127, 96]
    hq, hv = 2, 8
    T = sum(lens)
    q, k, v, g, b, S0 = _prefill_case(T, hq, hv, d, "bf16", 140, lens)
    cu = gdn_inputs.cu_from_lengths(lens)
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=chunk)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0), cu_seqlens=cu.numpy())
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill_many_heads[d={d},C={chunk}]", **e)
    assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16
