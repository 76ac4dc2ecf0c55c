"""gdn_prefill_noalloc (no workspace, no allocation inside the call: the
plan lives in a static per-GPU array) against gdn_prefill on the same
inputs, over calls in a row that reuse the static array with smaller inputs,
and against the fp64 oracle."""
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn
from oracle import gdn_oracle as orc
from parity import TOL_BF16, dev, np64, rel_err, report

pytestmark = pytest.mark.gpu


def _case(lens, hq, hv, d, seed):
    T = sum(lens)
    g0 = torch.Generator().manual_seed(seed)
    q = torch.randn((T, hq, d), generator=g0).to(torch.bfloat16)
    k = torch.randn((T, hq, d), generator=g0).to(torch.bfloat16)
    v = torch.randn((T, hv, d), generator=g0).to(torch.bfloat16)
    g = torch.nn.functional.logsigmoid(torch.randn((T, hv), generator=g0))
    b = torch.sigmoid(torch.randn((T, hv), generator=g0))
    S0 = 0.1 * torch.randn((len(lens), hv, d, d), generator=g0)
    cu = gdn_inputs.cu_from_lengths(lens) if len(lens) > 1 else None
    return q, k, v, g, b, S0, cu


def _both(lens, hq, hv, d, chunk, seed, emit_every=0):
    q, k, v, g, b, S0, cu = _case(lens, hq, hv, d, seed)
    args = (dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), dev(cu))
    ref = gdn.prefill(*args, chunk=chunk, emit_every=emit_every)
    o = torch.full_like(ref[0], float("nan"))
    S = torch.full_like(ref[1], float("nan"))
    cs = torch.full_like(ref[2], float("nan")) if emit_every else None
    gdn.prefill_noalloc(*args, o, S, chunk=chunk, emit_every=emit_every, chunk_states=cs)
    torch.cuda.synchronize()
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0),
                                  cu_seqlens=None if cu is None else cu.numpy())
    return ref, (o, S, cs), (ro, rS)


@pytest.mark.parametrize("d,chunk", [(128, 64), (64, 32)])
def test_noalloc_equals_fused_prefill_on_calls_in_a_row(monkeypatch, d, chunk):
    # both entry points on the fused kernel: the results must be identical
    monkeypatch.setenv("GDN_PREFILL_FUSED", "1")
    monkeypatch.delenv("GDN_FUSED_COLS", raising=False)
    calls = [([300, 0, 1, 517, 64, 200, 129], 2, 6, 2),  # emitting chunk states
             ([70, 33], 1, 3, 0),                          # smaller: a stale plan must not matter
             ([95], 1, 2, 0)]                              # one sequence: no plan at all
    for i, (lens, hq, hv, emit) in enumerate(calls):
        ref, got, (ro, rS) = _both(lens, hq, hv, d, chunk, 30 + i, emit)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
        if emit:
            assert torch.equal(got[2], ref[2])
        e = dict(o=rel_err(got[0], ro), state=rel_err(got[1], rS))
        report(f"noalloc[d={d},C={chunk}] call {i} lens {lens}", **e)
        assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16


def test_noalloc_matches_default_prefill():
    # gdn_prefill left to choose (the separate launches for so few pairs)
    for i, lens in enumerate(([1000, 3, 250], [129])):
        ref, got, _ = _both(lens, 2, 4, 128, 64, 40 + i)
        e = dict(o=rel_err(got[0], ref[0].double().cpu().numpy()), state=rel_err(got[1], ref[1].cpu().numpy()))
        report(f"noalloc vs gdn_prefill lens {lens}", **e)
        assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16
