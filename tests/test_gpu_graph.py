"""HIP graph capture of the prefill step (gdn_conv1d, then gdn_prefill): the
graphs are replayed several times, with eager calls on other buffers and
synchronisations between the replays, and every replay must reproduce the
eager result exactly (the kernels are deterministic).  Covers the split scan
with its join (one sequence), the one-pass scan and the planned varlen
path (cu_seqlens)."""
import pytest
import torch

import gdn_inputs
import linear_attention_token_conv1d_amd as gdn

pytestmark = pytest.mark.gpu


def _case(lens, h_qk, h_v, d, seed):
    T = sum(lens)
    C = 2 * h_qk * d + h_v * d
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn((T, C), generator=gen).to(torch.bfloat16).cuda()
    w = (0.5 * torch.randn((C, 4), generator=gen)).to(torch.bfloat16).cuda()
    g = torch.nn.functional.logsigmoid(torch.randn((T, h_v), generator=gen)).cuda()
    b = torch.sigmoid(torch.randn((T, h_v), generator=gen)).cuda()
    s0 = (0.1 * torch.randn((len(lens), h_v, d, d), generator=gen)).cuda()
    cu = gdn_inputs.cu_from_lengths(lens).cuda() if len(lens) > 1 else None
    return T, x, w, g, b, s0, cu


class _Step:
    """One prefill step on its own buffers."""

    def __init__(self, case, h_qk, h_v, d):
        self.T, self.x, self.w, self.g, self.b, self.s0, self.cu = case
        self.h_qk, self.h_v, self.d = h_qk, h_v, d
        n = 1 if self.cu is None else self.cu.numel() - 1
        self.y = torch.empty_like(self.x)
        self.o = torch.empty((self.T, h_v, d), dtype=torch.bfloat16, device="cuda")
        self.fs = torch.empty((n, h_v, d, d), dtype=torch.float32, device="cuda")
        self.q, self.k, self.v = gdn.split_qkv(self.y, h_qk, d, h_v, d)
        self.ws = torch.empty(max(1, gdn.prefill_workspace_size(self.q, self.v, n, 64)), dtype=torch.uint8,
                              device="cuda")

    def conv(self):
        gdn.conv1d(self.x, self.w, None, None, self.cu, "silu", out=self.y)

    def pre(self):
        gdn.prefill(self.q, self.k, self.v, self.g, self.b, self.s0, self.cu, 64, 1.0, True, True, o=self.o,
                    final_state=self.fs, workspace=self.ws)


@pytest.mark.parametrize("lens,h_qk,h_v", [
    ([2048], 4, 8),             # split scan + join
    ([700], 2, 6),              # one-pass scan, grouped heads
    ([300, 1, 0, 517, 64], 2, 4),  # varlen: plan + one-pass scan
])
def test_graph_replays_match_eager(lens, h_qk, h_v):
    d = 128
    st = _Step(_case(lens, h_qk, h_v, d, seed=11), h_qk, h_v, d)
    other = _Step(_case(lens, h_qk, h_v, d, seed=12), h_qk, h_v, d)
    st.conv(); st.pre()
    torch.cuda.synchronize()
    o_ref, fs_ref = st.o.clone(), st.fs.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.conv(); st.pre()
    torch.cuda.current_stream().wait_stream(side)
    g_conv, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_conv):
        st.conv()
    with torch.cuda.graph(g_pre):
        st.pre()
    for rep in range(4):
        st.o.fill_(float("nan"))
        st.fs.fill_(float("nan"))
        g_conv.replay()
        g_pre.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.o, o_ref), f"replay {rep}: o"
        assert torch.equal(st.fs, fs_ref), f"replay {rep}: final state"
        other.conv(); other.pre()  # eager work on other buffers between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("lens", [[2048], [300, 1, 0, 517, 64]])
def test_backward_graph_replays_match_eager(lens):
    """gdn_prefill_backward then gdn_conv1d_backward captured in one HIP graph
    (the workspace carries the chunk plan, so the varlen pack is covered),
    replayed with eager backward calls on other buffers in between."""
    h_qk, h_v, d = 2, 4, 128
    T, x, w, g, b, s0, cu = _case(lens, h_qk, h_v, d, seed=21)
    n = 1 if cu is None else cu.numel() - 1
    C = x.shape[1]
    y = gdn.conv1d(x, w, None, None, cu, "silu")
    q, k, v = gdn.split_qkv(y, h_qk, d, h_v, d)
    gen = torch.Generator().manual_seed(22)
    do = torch.randn((T, h_v, d), generator=gen).to(torch.bfloat16).cuda()
    dsf = (0.3 * torch.randn((n, h_v, d, d), generator=gen)).cuda()
    dy = torch.zeros_like(y)
    dq, dk, dv = gdn.split_qkv(dy, h_qk, d, h_v, d)
    dg = torch.empty((T, h_v), dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)
    ds0 = torch.empty((n, h_v, d, d), dtype=torch.float32, device="cuda")
    dx = torch.empty_like(x)
    ws = torch.empty(gdn.prefill_backward_workspace_size(q, v, n, 64), dtype=torch.uint8, device="cuda")
    cws = torch.empty(gdn.conv1d_backward_workspace_size(T, C), dtype=torch.uint8, device="cuda")
    outs = {}

    def step():
        gdn.prefill_backward(q, k, v, g, b, do, s0, dsf, cu, 64, dq=dq, dk=dk, dv=dv, dg=dg, dbeta=db,
                             d_initial_state=ds0, workspace=ws)
        outs["conv"] = gdn.conv1d_backward(x, w, dy, None, None, cu, "silu", None, dx=dx, d_conv_state=False,
                                           workspace=cws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dy, dg, db, ds0, dx, outs["conv"][1])]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (dg, db, ds0, dx):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = [dy, dg, db, ds0, dx, outs["conv"][1]]
        for i, (a, r) in enumerate(zip(got, ref)):
            assert torch.equal(a, r), f"replay {rep}: output {i}"
        # eager backward on other inputs between replays
        gdn.prefill_backward(q, k, v, g, b, torch.zeros_like(do), None, None, cu, 64)
        torch.cuda.synchronize()
