"""CPU checks of the C-ABI library: it loads, exports every function declared
in include/gdn.h, its argument structs match the header's layout (checked
with a C compiler), and host-side validation rejects bad arguments before
any launch (these calls never reach the GPU)."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import linear_attention_token_conv1d_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_ ]*?\**\s*(gdn_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"gdn_conv1d", "gdn_prefill", "gdn_decode_step", "gdn_prefill_workspace_size",
            "gdn_status_string", "gdn_last_error", "gdn_abi_version"} <= set(names)
    L = gdn.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), n
    assert L.gdn_abi_version() == gdn.ABI_VERSION == 4


def test_struct_layout_matches_header():
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "gdn.h"
#define P(s, f) printf(#s "." #f " %zu\n", offsetof(s, f))
int main(void) {
  printf("conv %zu\nprefill %zu\ndecode %zu\n", sizeof(gdn_conv1d_args), sizeof(gdn_prefill_args),
         sizeof(gdn_decode_args));
  P(gdn_conv1d_args, total_tokens); P(gdn_conv1d_args, cu_seqlens);
  P(gdn_prefill_args, total_tokens); P(gdn_prefill_args, scale); P(gdn_prefill_args, q_stride);
  P(gdn_prefill_args, workspace_bytes); P(gdn_decode_args, scale); P(gdn_decode_args, o);
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = dict(l.rsplit(" ", 1) for l in subprocess.run([exe], capture_output=True, text=True,
                                                               check=True).stdout.split("\n") if l)
    assert int(lines["conv"]) == ctypes.sizeof(gdn.ConvArgs)
    assert int(lines["prefill"]) == ctypes.sizeof(gdn.PrefillArgs)
    assert int(lines["decode"]) == ctypes.sizeof(gdn.DecodeArgs)
    for key, val in lines.items():
        if "." in key:
            s, f = key.split(".")
            cls = {"gdn_conv1d_args": gdn.ConvArgs, "gdn_prefill_args": gdn.PrefillArgs,
                   "gdn_decode_args": gdn.DecodeArgs}[s]
            assert getattr(cls, f).offset == int(val), key


def _prefill(**kw):
    base = dict(struct_size=ctypes.sizeof(gdn.PrefillArgs), io_dtype=1, n_seqs=1, total_tokens=64,
                h_qk=2, h_v=6, d_k=128, d_v=128, chunk=64, scale=1.0, q=0x1000, k=0x2000, v=0x3000,
                q_stride=256, k_stride=256, v_stride=768, g=0x4000, beta=0x5000, o=0x6000)
    base.update(kw)
    a = gdn.PrefillArgs(**base)
    st = gdn.lib().gdn_prefill(ctypes.byref(a), None)
    return st, gdn.lib().gdn_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(h_v=5), 1), (dict(d_k=96, d_v=96), 2), (dict(d_v=64), 2), (dict(chunk=48), 2),
    (dict(q=0), 1), (dict(n_seqs=0), 1), (dict(n_seqs=2), 1), (dict(io_dtype=7), 1),
    (dict(q_stride=100), 1), (dict(q_stride=260), 3), (dict(q=0x1001), 3), (dict(flags=8), 1),
    (dict(struct_size=8), 1), (dict(total_tokens=-1), 1),
    # fp32 at chunk 64 is supported for both head widths: only the workspace is missing
    (dict(io_dtype=0, d_k=128, d_v=128, chunk=64), 4), (dict(io_dtype=0, d_k=64, d_v=64, chunk=64), 4),
    (dict(emit_every=-1), 1), (dict(emit_every=2), 1), (dict(emit_every=2, chunk_states=0x7008), 3),
    (dict(state_idx=0x7002), 3), (dict(state_dtype=7), 1),
    # a struct of the previous ABI (no state_dtype) is read as fp32 states
    (dict(struct_size=gdn.PrefillArgs.state_dtype.offset), 4),
    (dict(struct_size=gdn.PrefillArgs.state_dtype.offset - 8), 1),
    # final_state may alias initial_state exactly, not partly
    (dict(initial_state=0x100000, final_state=0x100010), 1),
])
def test_prefill_validation(kw, code):
    st, msg = _prefill(**kw)
    assert st == code, msg
    assert msg.startswith("gdn_prefill")


def test_conv_and_decode_validation():
    L = gdn.lib()
    a = gdn.ConvArgs(struct_size=ctypes.sizeof(gdn.ConvArgs), dtype=1, n_seqs=1, channels=12,
                     total_tokens=4, width=4, activation=1, x=0x1000, weight=0x2000, y=0x3000)
    assert L.gdn_conv1d(ctypes.byref(a), None) == 2  # channels % 8
    a.channels, a.width = 16, 5
    assert L.gdn_conv1d(ctypes.byref(a), None) == 2
    a.width, a.y = 4, 0x1010  # y overlaps x
    assert L.gdn_conv1d(ctypes.byref(a), None) == 1
    assert b"overlap" in L.gdn_last_error()
    d = gdn.DecodeArgs(struct_size=ctypes.sizeof(gdn.DecodeArgs), io_dtype=1, state_dtype=1, n_seqs=4,
                       h_qk=2, h_v=6, d_k=128, d_v=128, width=4, activation=1, scale=1.0, x=0x1000,
                       conv_weight=0x2000, conv_state=0, g=0x3000, beta=0x4000, state=0x5000, o=0x6000)
    assert L.gdn_decode_step(ctypes.byref(d), None) == 1  # conv without a conv state
    d.conv_weight = 0
    d.h_qk, d.h_v = 1, 32
    assert L.gdn_decode_step(ctypes.byref(d), None) == 2  # more than 16 V heads per QK head
    d.h_qk, d.h_v, d.state = 2, 6, 0x5008
    assert L.gdn_decode_step(ctypes.byref(d), None) == 3
    d.state, d.conv_head = 0x5000, 0x7002
    assert L.gdn_decode_step(ctypes.byref(d), None) == 3  # misaligned ring heads
    a.conv_head = 0x7002
    assert L.gdn_conv1d(ctypes.byref(a), None) == 3
    # structs of the previous ABI (no conv_head) are accepted; shorter ones are not
    a.conv_head, a.y = 0, 0x3000
    a.struct_size = gdn.ConvArgs.conv_head.offset - 8
    assert L.gdn_conv1d(ctypes.byref(a), None) == 1
    d.struct_size = gdn.DecodeArgs.conv_head.offset - 8
    assert L.gdn_decode_step(ctypes.byref(d), None) == 1


def test_prefill_noalloc_validation():
    """gdn_prefill_noalloc checks its arguments like gdn_prefill (without the
    workspace) and rejects what the fused kernel and its static plan cannot
    take, before touching a GPU."""
    L = gdn.lib()

    def call(**kw):
        base = dict(struct_size=ctypes.sizeof(gdn.PrefillArgs), io_dtype=1, n_seqs=1, total_tokens=64,
                    h_qk=2, h_v=6, d_k=128, d_v=128, chunk=64, scale=1.0, q=0x1000, k=0x2000, v=0x3000,
                    q_stride=256, k_stride=256, v_stride=768, g=0x4000, beta=0x5000, o=0x6000)
        base.update(kw)
        a = gdn.PrefillArgs(**base)
        return L.gdn_prefill_noalloc(ctypes.byref(a), None), L.gdn_last_error().decode()

    assert call(io_dtype=0)[0] == 2 and "bf16" in call(io_dtype=0)[1]
    assert call(chunk=16)[0] == 2
    st, msg = call(n_seqs=gdn.NOALLOC_MAX_SEQS + 1, cu_seqlens=0x8000)
    assert st == 1 and "static plan" in msg
    assert call(h_v=5)[0] == 1 and call(q=0x1001)[0] == 3 and call(emit_every=2)[0] == 1


def test_prefill_requires_workspace():
    st, msg = _prefill()
    assert st == 4 and "workspace" in msg
    st, msg = _prefill(workspace=0x10000, workspace_bytes=16)
    assert st == 4


def test_workspace_size_query():
    a = gdn.PrefillArgs(struct_size=ctypes.sizeof(gdn.PrefillArgs), n_seqs=1, total_tokens=1024, h_qk=16,
                        h_v=48, d_k=128, d_v=128, chunk=64)
    a.io_dtype = 1
    n = gdn.lib().gdn_prefill_workspace_size(ctypes.byref(a))
    # one sequence of 48 heads runs the separate preparation and scan: offsets
    # + (1024/64 + 1) chunks x 48 heads x (Tb + P in the io dtype + 4 fp32 rows)
    assert n == 256 + 17 * 48 * (2 * 64 * 64 * 2 + 16 * 64)
    # 100 sequences run the fused kernel: only the plan's arrays (chunk
    # offsets, scan order, emitted-state rows), padded to 256 bytes
    a.n_seqs = 100
    assert gdn.lib().gdn_prefill_workspace_size(ctypes.byref(a)) == (100 * 3 + 2) * 4 // 256 * 256 + 256
    a.n_seqs, a.io_dtype = 1, 0
    n = gdn.lib().gdn_prefill_workspace_size(ctypes.byref(a))
    assert n == 256 + 17 * 48 * (2 * 64 * 64 * 4 + 16 * 64)
    assert gdn.lib().gdn_status_string(5) == b"GDN_ERR_HIP"


@pytest.mark.parametrize("cname,pyt", [("gdn_prefill_backward_args", "PrefillBwdArgs"),
                                       ("gdn_conv1d_backward_args", "ConvBwdArgs"),
                                       ("gdn_prefill_args", "PrefillArgs"), ("gdn_conv1d_args", "ConvArgs"),
                                       ("gdn_decode_args", "DecodeArgs")])
def test_every_field_offset_matches_header(cname, pyt):
    """Every field of the binding's ctypes struct sits at the header's offset."""
    st = getattr(gdn, pyt)
    lines = [f'printf("size %zu\\n", sizeof({cname}));']
    lines += [f'printf("{f} %zu\\n", offsetof({cname}, {f}));' for f, _ in st._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"gdn.h\"\nint main(void) {\n" + "\n".join(lines) + \
        "\nreturn 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = dict(l.split(" ") for l in subprocess.run([exe], capture_output=True, text=True,
                                                         check=True).stdout.split("\n") if l)
    assert int(got["size"]) == ctypes.sizeof(st)
    for f, _ in st._fields_:
        assert int(got[f]) == getattr(st, f).offset, f


def _bwd_args(**kw):
    a = gdn.PrefillBwdArgs(struct_size=ctypes.sizeof(gdn.PrefillBwdArgs), flags=1, io_dtype=1, n_seqs=1,
                           total_tokens=128, h_qk=2, h_v=4, d_k=64, d_v=64, chunk=64, scale=1.0)
    base = 1 << 32
    for i, f in enumerate(["q", "k", "v", "g", "beta", "d_o", "dq", "dk", "dv", "dg", "dbeta"]):
        setattr(a, f, base + i * (1 << 24))
    a.q_stride = a.k_stride = a.dq_stride = a.dk_stride = 128
    a.v_stride = a.dv_stride = 256
    a.workspace = 1 << 40
    a.workspace_bytes = gdn.lib().gdn_prefill_backward_workspace_size(ctypes.byref(a))
    for f, v in kw.items():
        setattr(a, f, v)
    return a


def test_prefill_backward_validation():
    """Host-side rejections of gdn_prefill_backward (no launch: the pointers are never touched)."""
    L = gdn.lib()
    call = lambda a: L.gdn_prefill_backward(ctypes.byref(a), None)
    assert _bwd_args().workspace_bytes > 0
    assert call(_bwd_args(d_k=96, d_v=96)) == 2
    assert call(_bwd_args(chunk=48)) == 2
    assert call(_bwd_args(h_v=3)) == 1
    assert call(_bwd_args(flags=8)) == 1
    assert call(_bwd_args(d_o=0)) == 1
    assert call(_bwd_args(n_seqs=2)) == 1  # cu_seqlens missing
    assert call(_bwd_args(dq_stride=64)) == 1
    assert call(_bwd_args(dq=(1 << 32) + 8)) == 3
    assert call(_bwd_args(dv_stride=260)) == 3
    assert call(_bwd_args(dk=(1 << 32) + 16)) == 1  # dk overlaps q
    a = _bwd_args()
    a.workspace_bytes -= 1
    assert call(a) == 4
    assert call(_bwd_args(workspace=(1 << 40) + 16)) == 3
    a = _bwd_args(struct_size=8)
    assert call(a) == 1
    # one sequence past the budget runs in windows: the workspace is bounded
    # by the budget (down to windows of one chunk); a varlen pack past it runs
    # its sequences one by one in a workspace of the budget
    big = dict(total_tokens=65536, h_qk=16, h_v=48, d_k=128, d_v=128)
    assert L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(**big))) <= 4 << 30
    assert L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(n_seqs=2, cu_seqlens=0x100, **big))) == 4 << 30
    pack = dict(total_tokens=262144, h_qk=16, h_v=48, d_k=128, d_v=128, n_seqs=8, cu_seqlens=0x100)
    assert L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(**pack))) == 4 << 30
    # a pack within the budget keeps its whole-call workspace
    small = dict(total_tokens=512, n_seqs=3, cu_seqlens=0x100)
    assert 0 < L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(**small))) < 4 << 30
    # the workspace grows with the chunk count and the heads
    s1 = L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(total_tokens=1024)))
    s2 = L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(total_tokens=2048)))
    assert s2 > s1 > 0
    assert L.gdn_prefill_backward_workspace_size(ctypes.byref(_bwd_args(d_k=96, d_v=96))) == 0


def test_conv1d_backward_validation():
    L = gdn.lib()
    def args(**kw):
        a = gdn.ConvBwdArgs(struct_size=ctypes.sizeof(gdn.ConvBwdArgs), dtype=1, n_seqs=1, channels=64,
                            total_tokens=100, width=4, activation=1)
        base = 1 << 32
        for i, f in enumerate(["x", "weight", "dy", "dx", "dweight"]):
            setattr(a, f, base + i * (1 << 24))
        a.workspace = 1 << 40
        a.workspace_bytes = L.gdn_conv1d_backward_workspace_size(ctypes.byref(a))
        for f, v in kw.items():
            setattr(a, f, v)
        return a
    call = lambda a: L.gdn_conv1d_backward(ctypes.byref(a), None)
    assert args().workspace_bytes >= 2 * 64 * 5 * 4
    assert call(args(width=5)) == 2
    assert call(args(activation=7)) == 1
    assert call(args(dy=0)) == 1
    assert call(args(dbias=(1 << 32) + (6 << 24))) == 1  # dbias without bias
    assert call(args(dx=(1 << 32) + 64)) == 1  # dx overlaps x
    assert call(args(n_seqs=3)) == 1
    assert call(args(channels=60)) == 2
    assert call(args(dy=(1 << 32) + (2 << 24) + 8)) == 3
    a = args()
    a.workspace_bytes = 16
    assert call(a) == 4
