"""The fused prefill kernel (one launch: each chunk's preparation folded into
the scan) at all three workgroup widths, 16, 32 and 64 d_v columns.

gdn_prefill takes the fused kernel by itself only when its 64-column
workgroups fill the chip (many sequence x V-head pairs); the small cases of
the other GPU test files then run the separate preparation and scan.  Here
GDN_PREFILL_FUSED=1 and GDN_FUSED_COLS force the fused kernel and a width,
and the bf16 cases at chunk 32 and 64 of those files run again under each:
ragged tails, varlen packs with empty and one-token sequences, state slots,
emitted chunk states, bf16 states, erase off, no L2 norm, strided and in-place
tensors, the conv + prefill layer and graph replays.  Every case compares
with the fp64 oracle (or with eager results) as in its own file."""
import numpy as np
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn
import test_gpu_boundary as boundary
import test_gpu_graph as graph
import test_gpu_small as small
from oracle import gdn_oracle as orc
from parity import TOL_BF16, dev, np64, rel_err, report

pytestmark = pytest.mark.gpu

CASES = [
    ("ragged_128_64", small.test_prefill_ragged, dict(io="bf16", d=128, chunk=64)),
    ("ragged_128_32", small.test_prefill_ragged, dict(io="bf16", d=128, chunk=32)),
    ("ragged_64_64", small.test_prefill_ragged, dict(io="bf16", d=64, chunk=64)),
    ("erase_off_ragged", small.test_prefill_erase_off, dict(io="bf16", d=128, chunk=64, T=201, lens=None)),
    ("erase_off_varlen", small.test_prefill_erase_off, dict(io="bf16", d=64, chunk=32, T=None, lens=[40, 0, 130, 7])),
    ("emission_varlen", small.test_prefill_chunk_state_emission,
     dict(io="bf16", d=128, chunk=64, K=1, lens=[200, 0, 300, 64, 65])),
    ("emission_long", small.test_prefill_chunk_state_emission, dict(io="bf16", d=128, chunk=64, K=2, lens=[2500])),
    ("state_slots", small.test_prefill_state_slots, dict(lens=[70, 130, 5], slots=[2, 0, 3], pool=4)),
    ("degenerate_lengths", small.test_prefill_varlen_degenerate_lengths, dict(io="bf16")),
    ("no_l2norm_scale", small.test_prefill_no_l2norm_and_scale, {}),
    ("in_place_strided", small.test_prefill_in_place_state_and_strided_inputs, {}),
    ("layer", small.test_layer_conv_then_prefill, {}),
    ("many_heads_128_32", small.test_prefill_many_heads_wider_blocks, dict(d=128, chunk=32)),
    ("many_heads_64_64", small.test_prefill_many_heads_wider_blocks, dict(d=64, chunk=64)),
    ("bf16_states_varlen", boundary.test_prefill_bf16_states, dict(io="bf16", d=128, chunk=64, lens=[0, 1, 70, 200])),
    ("bf16_states_32", boundary.test_prefill_bf16_states, dict(io="bf16", d=64, chunk=32, lens=[300])),
    ("bf16_chunk_states_in_place", boundary.test_prefill_bf16_chunk_states_and_in_place, {}),
    ("graph_varlen", graph.test_graph_replays_match_eager, dict(lens=[300, 1, 0, 517, 64], h_qk=2, h_v=4)),
    ("graph_long", graph.test_graph_replays_match_eager, dict(lens=[700], h_qk=2, h_v=6)),
]


@pytest.mark.parametrize("cols", ["16", "32", "64", "wide"])
@pytest.mark.parametrize("name,fn,kw", CASES, ids=[c[0] for c in CASES])
def test_fused_kernel_width(monkeypatch, cols, name, fn, kw):
    monkeypatch.setenv("GDN_PREFILL_FUSED", "1")
    monkeypatch.setenv("GDN_FUSED_COLS", cols)
    fn(**kw)


def test_fused_kernel_chosen_for_many_pairs(monkeypatch):
    """Without the switches: 40 sequences x 8 V heads at d 128 fill the chip
    with 64-column workgroups, so the call runs the fused kernel, whose
    workspace is the plan's arrays only."""
    monkeypatch.delenv("GDN_PREFILL_FUSED", raising=False)
    monkeypatch.delenv("GDN_FUSED_COLS", raising=False)
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(0, 160, size=40)]
    lens[3], lens[11] = 0, 1
    hq, hv, d = 2, 8, 128
    T = sum(lens)
    q, k, v, g, b, S0 = small._prefill_case(T, hq, hv, d, "bf16", 170, lens)
    cu = gdn_inputs.cu_from_lengths(lens)
    assert gdn.prefill_workspace_size(dev(q), dev(v), n_seqs=len(lens), chunk=64) < 4096
    o, S = gdn.prefill(dev(q), dev(k), dev(v), dev(g), dev(b), dev(S0), cu_seqlens=dev(cu), chunk=64)
    ro, rS = orc.gated_delta_rule(np64(q), np64(k), np64(v), np64(g), np64(b), np64(S0), cu_seqlens=cu.numpy())
    e = dict(o=rel_err(o, ro), state=rel_err(S, rS))
    report("fused_auto[40 seqs x 8 heads]", **e)
    assert e["o"] < TOL_BF16 and e["state"] < TOL_BF16
