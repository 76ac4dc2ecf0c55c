"""GPU parity of the boundary options against the fp64 oracle: conv-state ring
heads (gdn_conv1d reads a ring and leaves the state chronological; a decode
step overwrites one slot and advances the head), prefill states stored as
bf16 or fp32 (initial, final and chunk-boundary states), and fp32 prefill at
chunk 64."""
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


# ------------------------------------------------------------ ring heads

@pytest.mark.parametrize("io,width", [("bf16", 4), ("f32", 3), ("bf16", 2)])
def test_conv1d_reads_ring_and_resets_heads(io, width):
    lens = [5, 1, 0, 2, 130, 3, 64]
    N, T, C = len(lens), sum(lens), 2056  # several workgroups per sequence in the state pass
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((T, C), DT[io], seed=1)
    w = _rand((C, width), DT[io], 0.5, seed=2)
    ring = _rand((N, C, width - 1), DT[io], seed=3)
    heads = torch.tensor([n % (width - 1) for n in range(N)], dtype=torch.int32)
    chrono = orc.ring_to_chronological(np64(ring), heads.numpy())
    st_d, hd_d = dev(ring.clone()), dev(heads.clone())
    y = gdn.conv1d(dev(x), dev(w), None, st_d, dev(cu), conv_head=hd_d)
    ry, rst = orc.causal_conv1d(np64(x), np64(w), None, chrono, cu.numpy())
    e_y = rel_err(y, ry)
    report(f"conv1d_ring[{io},W={width}]", y=e_y)
    assert e_y < (4e-3 if io == "bf16" else 1e-6)
    assert np.array_equal(np64(st_d), rst)  # chronological on return, bit for bit
    assert bool((hd_d == 0).all())


@pytest.mark.parametrize("io,state_dt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_decode_ring_writes_one_slot(io, state_dt):
    """Six decode steps on a ring: every step overwrites exactly the slot at
    the head with the new input, leaves the other slots' bits alone and
    advances the head; outputs and states follow the oracle run on the
    chronological conv state, with state slots (state_idx) in play."""
    N, hq, hv, d, W, steps = 5, 2, 6, 128, 4, 6
    C = 2 * hq * d + hv * d
    pool = 7
    idx = torch.tensor([4, 0, 6, 2, 5], dtype=torch.int32)
    w = _rand((C, W), DT[io], 0.5, seed=8)
    ring = _rand((pool, C, W - 1), DT[io], seed=9)
    heads = torch.tensor([s % (W - 1) for s in range(pool)], dtype=torch.int32)
    S = _rand((pool, hv, d, d), DT[state_dt], 0.1, seed=10)
    S_d, ring_d, hd_d = dev(S.clone()), dev(ring.clone()), dev(heads.clone())
    il = idx.long()
    rS = np64(S[il])
    rcs = orc.ring_to_chronological(np64(ring[il]), heads[il].numpy())
    tol = TOL_BF16 if "bf16" in (io, state_dt) else TOL_F32
    worst = 0.0
    for t in range(steps):
        x = _rand((N, C), DT[io], seed=100 + t)
        g, b = _gates(N, hv, 200 + t)
        before = ring_d.clone()
        h_before = hd_d.clone()
        o = gdn.decode_step(dev(x), dev(g), dev(b), S_d, hq, hv, d, conv_weight=dev(w), conv_state=ring_d,
                            state_idx=dev(idx), conv_head=hd_d)
        ro, rS, rcs = orc.decode_step(np64(x), np64(w), np64(g), np64(b), rS, rcs, hq, d, hv, d)
        worst = max(worst, rel_err(o, ro))
        torch.cuda.synchronize()
        for n in range(N):
            s, h = int(idx[n]), int(h_before[int(idx[n])])
            changed = (ring_d[s] != before[s]).any(dim=0)  # per slot
            assert torch.equal(ring_d[s, :, h].cpu(), x[n]), (t, n)
            assert not bool(changed[[j for j in range(W - 1) if j != h]].any()), (t, n)
            assert int(hd_d[s]) == (h + 1) % (W - 1)
        untouched = [s for s in range(pool) if s not in idx.tolist()]
        assert torch.equal(ring_d[untouched].cpu(), ring[untouched]) and torch.equal(hd_d[untouched].cpu(), heads[untouched])
    got = orc.ring_to_chronological(np64(ring_d[il]), hd_d[il].cpu().numpy())
    e = dict(o=worst, state=rel_err(S_d[il], rS))
    report(f"decode_ring[{io},{state_dt}]", **e)
    assert np.array_equal(got, rcs)
    assert e["o"] < tol and e["state"] < tol


def test_layer_ring_then_decode():
    """A ring left by decode steps feeds a prefill conv (read in ring order,
    written back chronological with the head at 0), and decode continues on
    it: the outputs equal the oracle over the same token stream."""
    N, hq, hv, d, W = 3, 1, 3, 64, 4
    C = 2 * hq * d + hv * d
    w = _rand((C, W), torch.float32, 0.5, seed=30)
    ring = _rand((N, C, W - 1), torch.float32, seed=31)
    heads = torch.tensor([2, 0, 1], dtype=torch.int32)
    ring_d, hd_d = dev(ring.clone()), dev(heads.clone())
    rcs = orc.ring_to_chronological(np64(ring), heads.numpy())
    lens = [9, 1, 4]
    cu = gdn_inputs.cu_from_lengths(lens)
    x = _rand((sum(lens), C), torch.float32, seed=32)
    y = gdn.conv1d(dev(x), dev(w), None, ring_d, dev(cu), conv_head=hd_d)
    ry, rcs = orc.causal_conv1d(np64(x), np64(w), None, rcs, cu.numpy())
    assert rel_err(y, ry) < 1e-6 and bool((hd_d == 0).all())
    S = dev(torch.zeros((N, hv, d, d)))
    rS = np.zeros((N, hv, d, d))
    for t in range(4):
        xt = _rand((N, C), torch.float32, seed=40 + t)
        g, b = _gates(N, hv, 50 + t)
        o = gdn.decode_step(dev(xt), dev(g), dev(b), S, hq, hv, d, conv_weight=dev(w), conv_state=ring_d,
                            conv_head=hd_d)
        ro, rS, rcs = orc.decode_step(np64(xt), np64(w), np64(g), np64(b), rS, rcs, hq, d, hv, d)
        assert rel_err(o, ro) < TOL_F32
    assert np.array_equal(orc.ring_to_chronological(np64(ring_d), hd_d.cpu().numpy()), rcs)


# ------------------------------------------------------- prefill state dtype

def _case(T, hq, hv, d, io, seed, N):
    q = _rand((T, hq, d), DT[io], seed=seed)
    k = _rand((T, hq, d), DT[io], seed=seed + 1)
    v = _rand((T, hv, d), DT[io], seed=seed + 2)
    g, b = _gates(T, hv, seed + 3)
    S0 = _rand((N, hv, d, d), torch.float32, 0.1, seed=seed + 4)
    return q, k, v, g, b, S0


@pytest.mark.parametrize("io,d,chunk,lens", [
    ("bf16", 128, 64, [0, 1, 70, 200]),   # varlen, empty and 1-token sequences
    ("bf16", 64, 32, [300]),
    ("f32", 64, 16, [40, 90]),             # fp32 scan
    ("bf16", 128, 64, [2500]),             # one long sequence (split scan and join)
])
def test_prefill_bf16_states(io, d, chunk, lens):
    """initial_state and final_state stored as bf16: read exactly, written
    with round-to-nearest-even; the oracle starts from the same bf16 values."""
    hq, hv = 2, 4
    N, T = len(lens), sum(lens)
    q, k, v, g, b, S0 = _case(T, hq, hv, d, io, 60, N)
    S0b = S0.to(torch.bfloat16)
    cu = gdn_inputs.cu_from_lengths(lens) if N > 1 else None
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0b), cu_seqlens=dev(cu), chunk=chunk)
    assert S.dtype == torch.bfloat16
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0b),
                                  cu_seqlens=None if cu is None else cu.numpy())
    tol = TOL_BF16 if io == "bf16" else 4e-3  # fp32 io: the bf16 store of S dominates
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill_bf16_states[{io},d={d},C={chunk},{lens}]", **e)
    assert e["o"] < tol and e["state"] < tol
    # the final state is the fp32 result rounded once: compare with an fp32-state call
    _, S32 = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0b.float()), cu_seqlens=dev(cu),
                         chunk=chunk)
    assert torch.equal(S, S32.to(torch.bfloat16))


def test_prefill_bf16_chunk_states_and_in_place():
    """Chunk-boundary states in bf16, and a bf16 state updated in place
    (final_state aliasing initial_state)."""
    hq, hv, d, chunk, K = 2, 4, 128, 64, 2
    lens = [300, 129]
    T = sum(lens)
    q, k, v, g, b, S0 = _case(T, hq, hv, d, "bf16", 70, len(lens))
    S0b = S0.to(torch.bfloat16)
    cu = gdn_inputs.cu_from_lengths(lens)
    Sd = dev(S0b.clone())
    o, S, E = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), Sd, cu_seqlens=dev(cu), chunk=chunk,
                          final_state=Sd, emit_every=K)
    assert E.dtype == torch.bfloat16 and S.data_ptr() == Sd.data_ptr()
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0b), cu_seqlens=cu.numpy())
    assert rel_err(o, ro) < TOL_BF16 and rel_err(Sd, rS) < TOL_BF16
    r = 0
    for n, L in enumerate(lens):
        s0 = int(cu[n])
        for j in range(1, (L - 1) // (K * chunk) + 1):
            e = s0 + j * K * chunk
            _, rSj = orc.gated_delta_rule(np64(q[s0:e]), np64(k[s0:e]), np64(v[s0:e]), np64(g[s0:e]),
                                          np64(b[s0:e]), np64(S0b[n:n + 1]))
            assert rel_err(E[r:r + 1], rSj) < TOL_BF16
            r += 1
    assert r == E.shape[0]


# ------------------------------------------------------------ fp32 chunk 64

@pytest.mark.parametrize("d,lens", [(128, [0, 150, 64, 1]), (64, [333]), (128, [200])])
def test_prefill_fp32_chunk64(d, lens):
    """fp32 io at chunk 64 for both head widths (one chunk buffer in LDS)."""
    hq, hv = 2, 4
    N, T = len(lens), sum(lens)
    q, k, v, g, b, S0 = _case(T, hq, hv, d, "f32", 80, N)
    cu = gdn_inputs.cu_from_lengths(lens) if N > 1 else None
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=64)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0),
                                  cu_seqlens=None if cu is None else cu.numpy())
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report(f"prefill_f32_C64[d={d},{lens}]", **e)
    assert e["o"] < TOL_F32 and e["state"] < TOL_F32
    # the result does not depend on the chunk beyond rounding
    o16, S16 = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=16)
    assert rel_err(o, o16.double().cpu().numpy()) < TOL_F32
