"""Gated DeltaNet token mixer on MI355X (gfx950): Python binding of libgdn.so.

This module only marshals arguments: it checks torch-level properties
(device, dtype, contiguity), fills the C argument structs declared in
include/gdn.h and calls the library on torch's current HIP stream.  Every
step of the computation runs in the library's HIP kernels.  There is no
fallback: if libgdn.so is missing or fails to load, every call raises.

Entry points (same names as the C ABI):
    conv1d       causal depthwise conv (+ SiLU) with per-sequence conv state
    prefill      chunked gated delta rule over packed sequences
    decode_step  one token per sequence: conv step + recurrence, state in place
    prefill_backward, conv1d_backward   gradients of prefill and conv1d
and gdn_layer / gdn_layer_backward, which chain them for a whole token mixer
layer.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["conv1d", "prefill", "decode_step", "gdn_layer", "prefill_workspace_size", "lib",
           "prefill_backward", "conv1d_backward", "gdn_layer_backward", "GdnError", "LIB_PATH",
           "probe_mfma", "probe_copy", "prefill_noalloc", "NOALLOC_MAX_SEQS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

F32, BF16 = 0, 1
ACT_NONE, ACT_SILU = 0, 1
FLAG_L2NORM_QK = 1
FLAG_NO_ERASE = 2
ABI_VERSION = 4  # the gdn.h this binding matches
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_c_void_p = ctypes.c_void_p


class GdnError(RuntimeError):
    pass


class ConvArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("width", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("x", _c_void_p), ("weight", _c_void_p),
                ("bias", _c_void_p), ("y", _c_void_p), ("conv_state", _c_void_p),
                ("cu_seqlens", _c_void_p), ("conv_head", _c_void_p)]


class PrefillArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("io_dtype", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("h_qk", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("scale", ctypes.c_float), ("q", _c_void_p),
                ("k", _c_void_p), ("v", _c_void_p), ("q_stride", ctypes.c_int64),
                ("k_stride", ctypes.c_int64), ("v_stride", ctypes.c_int64), ("g", _c_void_p),
                ("beta", _c_void_p), ("initial_state", _c_void_p), ("final_state", _c_void_p),
                ("o", _c_void_p), ("cu_seqlens", _c_void_p), ("workspace", _c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("emit_every", ctypes.c_int32),
                ("chunk_states", _c_void_p), ("state_idx", _c_void_p), ("state_dtype", ctypes.c_int32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("io_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
                ("n_seqs", ctypes.c_int32), ("h_qk", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("width", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("scale", ctypes.c_float), ("x", _c_void_p),
                ("conv_weight", _c_void_p), ("conv_bias", _c_void_p), ("conv_state", _c_void_p),
                ("g", _c_void_p), ("beta", _c_void_p), ("state", _c_void_p), ("o", _c_void_p),
                ("state_idx", _c_void_p), ("conv_head", _c_void_p)]


_lib = None


class PrefillBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("io_dtype", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("h_qk", ctypes.c_int32), ("h_v", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("q", _c_void_p), ("k", _c_void_p), ("v", _c_void_p),
                ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64), ("v_stride", ctypes.c_int64),
                ("g", _c_void_p), ("beta", _c_void_p), ("initial_state", _c_void_p),
                ("cu_seqlens", _c_void_p), ("d_o", _c_void_p), ("d_final_state", _c_void_p),
                ("dq", _c_void_p), ("dk", _c_void_p), ("dv", _c_void_p),
                ("dq_stride", ctypes.c_int64), ("dk_stride", ctypes.c_int64), ("dv_stride", ctypes.c_int64),
                ("dg", _c_void_p), ("dbeta", _c_void_p), ("d_initial_state", _c_void_p),
                ("workspace", _c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class ConvBwdArgs(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("dtype", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("total_tokens", ctypes.c_int64), ("width", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("x", _c_void_p), ("weight", _c_void_p),
                ("bias", _c_void_p), ("conv_state", _c_void_p), ("cu_seqlens", _c_void_p),
                ("dy", _c_void_p), ("d_new_state", _c_void_p), ("dx", _c_void_p), ("dweight", _c_void_p),
                ("dbias", _c_void_p), ("d_conv_state", _c_void_p), ("workspace", _c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


def lib():
    """The loaded libgdn.so (raises GdnError when it is missing or unloadable)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GdnError(f"{LIB_PATH} is not built; run python -m linear_attention_token_conv1d_amd._build")
        L = ctypes.CDLL(LIB_PATH)
        for name, argt in (("gdn_conv1d", ConvArgs), ("gdn_prefill", PrefillArgs),
                           ("gdn_prefill_noalloc", PrefillArgs), ("gdn_decode_step", DecodeArgs), ("gdn_prefill_backward", PrefillBwdArgs),
                           ("gdn_conv1d_backward", ConvBwdArgs)):
            f = getattr(L, name)
            f.argtypes = [ctypes.POINTER(argt), _c_void_p]
            f.restype = ctypes.c_int
        for name, argt in (("gdn_prefill_workspace_size", PrefillArgs),
                           ("gdn_prefill_backward_workspace_size", PrefillBwdArgs),
                           ("gdn_conv1d_backward_workspace_size", ConvBwdArgs)):
            f = getattr(L, name)
            f.argtypes = [ctypes.POINTER(argt)]
            f.restype = ctypes.c_size_t
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.gdn_probe_mfma_flops.restype = ctypes.c_int64
        L.gdn_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, _c_void_p, _c_void_p]
        L.gdn_probe_mfma.restype = ctypes.c_int
        L.gdn_probe_copy.argtypes = [_c_void_p, _c_void_p, ctypes.c_size_t, _c_void_p]
        L.gdn_probe_copy.restype = ctypes.c_int
        if L.gdn_abi_version() != ABI_VERSION:
            raise GdnError("libgdn.so ABI version mismatch")
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        L = lib()
        raise GdnError(f"{what}: {L.gdn_status_string(status).decode()}: {L.gdn_last_error().decode()}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise GdnError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _contig(t, name, dtype=None):
    _dev(t, name, dtype)
    if not t.is_contiguous():
        raise GdnError(f"{name} must be contiguous")
    return t


def _cu(cu_seqlens, n_tokens):
    if cu_seqlens is None:
        return None, 1
    _contig(cu_seqlens, "cu_seqlens", torch.int32)
    return cu_seqlens, cu_seqlens.numel() - 1


def conv1d(x, weight, bias=None, conv_state=None, cu_seqlens=None, activation="silu", out=None,
           conv_head=None):
    """Causal depthwise conv over packed sequences: x [T, C] -> y [T, C].

    weight [C, W]; conv_state [N, C, W-1] is read and then updated in place
    (None: zero history, nothing written).  conv_head [N] int32: the state's
    ring heads (slot of the oldest input); on return the state is
    chronological and the heads are 0."""
    _contig(x, "x")
    T, C = x.shape
    _contig(weight, "weight", x.dtype)
    if bias is not None:
        _contig(bias, "bias", x.dtype)
    if conv_state is not None:
        _contig(conv_state, "conv_state", x.dtype)
    if conv_head is not None:
        _contig(conv_head, "conv_head", torch.int32)
    cu, N = _cu(cu_seqlens, T)
    y = torch.empty_like(x) if out is None else _contig(out, "out", x.dtype)
    a = ConvArgs(ctypes.sizeof(ConvArgs), _DT[x.dtype], N, C, T, weight.shape[1],
                 ACT_SILU if activation == "silu" else ACT_NONE, _ptr(x), _ptr(weight), _ptr(bias),
                 _ptr(y), _ptr(conv_state), _ptr(cu), _ptr(conv_head))
    _check(lib().gdn_conv1d(ctypes.byref(a), _stream(x.device)), "gdn_conv1d")
    return y


def _prefill_args(q, k, v, g, beta, initial_state, final_state, o, cu, N, chunk, scale, l2norm,
                  workspace=None, erase=True, emit_every=0, chunk_states=None, state_idx=None,
                  state_dtype=torch.float32):
    T, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    flags = (FLAG_L2NORM_QK if l2norm else 0) | (0 if erase else FLAG_NO_ERASE)
    a = PrefillArgs(ctypes.sizeof(PrefillArgs), flags, _DT[q.dtype], N, T,
                    h_qk, h_v, d_k, d_v, chunk, scale, _ptr(q), _ptr(k), _ptr(v), q.stride(0),
                    k.stride(0), v.stride(0), _ptr(g), _ptr(beta), _ptr(initial_state),
                    _ptr(final_state), _ptr(o), _ptr(cu), _ptr(workspace),
                    0 if workspace is None else workspace.numel(), emit_every, _ptr(chunk_states),
                    _ptr(state_idx), _DT[state_dtype])
    return a


def prefill_workspace_size(q, v, n_seqs=1, chunk=64, emit_every=0):
    T, h_qk, d_k = q.shape
    a = PrefillArgs(struct_size=ctypes.sizeof(PrefillArgs), io_dtype=_DT[q.dtype], n_seqs=n_seqs,
                    total_tokens=T, h_qk=h_qk, h_v=v.shape[1], d_k=d_k, d_v=v.shape[2], chunk=chunk,
                    emit_every=emit_every)
    return lib().gdn_prefill_workspace_size(ctypes.byref(a))


def chunk_state_rows(lengths, chunk, emit_every):
    """Rows of chunk_states for sequences of these lengths: each sequence
    emits the state after every emit_every-th whole chunk that ends inside it
    (floor((len - 1) / (emit_every chunk)) states), in sequence order."""
    every = emit_every * chunk
    return sum((int(L) - 1) // every for L in lengths if int(L) > 0)


def _head_view(t, name, heads_dim_ok=True):
    """q/k/v: [T, H, d] with heads contiguous inside a token (token stride free)."""
    _dev(t, name)
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise GdnError(f"{name} must be [T, H, d] with contiguous heads")
    return t


def prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, chunk=64, scale=1.0,
            l2norm=True, output_final_state=True, o=None, final_state=None, workspace=None,
            erase=True, emit_every=0, chunk_states=None, state_idx=None, state_dtype=None):
    """Chunked gated delta rule.  q, k [T, H_qk, d], v [T, H_v, d] (bf16 or fp32,
    token stride free), g, beta [T, H_v] fp32, initial_state [N, H_v, d, d].
    erase=False runs the erase-off variant S_t = a_t S_{t-1} + b_t v_t k_t^T.
    emit_every=K > 0 also returns the chunk-boundary states [rows, H_v, d, d]
    (see chunk_state_rows) as a third result.  state_idx [N] int32 maps each
    sequence to a slot of the initial_state / final_state pools (both then
    given by the caller).  state_dtype (torch.float32 or torch.bfloat16; by
    default that of the state tensors passed, else fp32) is the dtype of the
    initial, final and chunk-boundary states in memory.

    Returns (o [T, H_v, d], final_state [N, H_v, d, d] or None)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _head_view(t, nm)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError("q, k and v must share a dtype")
    T = q.shape[0]
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    cu, N = _cu(cu_seqlens, T)
    h_v, d_v = v.shape[1], v.shape[2]
    if state_dtype is None:
        given = [t for t in (initial_state, final_state, chunk_states) if t is not None]
        state_dtype = given[0].dtype if given else torch.float32
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise GdnError("state_dtype must be torch.float32 or torch.bfloat16")
    for t, nm in ((initial_state, "initial_state"), (final_state, "final_state"), (chunk_states, "chunk_states")):
        if t is not None:
            _contig(t, nm, state_dtype)
    if o is None:
        o = torch.empty((T, h_v, d_v), dtype=q.dtype, device=q.device)
    if state_idx is not None:
        _contig(state_idx, "state_idx", torch.int32)
        if output_final_state and final_state is None:
            raise GdnError("with state_idx, pass the final_state pool")
    if output_final_state and final_state is None:
        final_state = torch.empty((N, h_v, d_v, q.shape[2]), dtype=state_dtype, device=q.device)
    if emit_every > 0 and chunk_states is None:
        lengths = [T] if cu is None else (cu[1:] - cu[:-1]).tolist()
        rows = chunk_state_rows(lengths, chunk, emit_every)
        chunk_states = torch.empty((max(rows, 1), h_v, d_v, q.shape[2]), dtype=state_dtype, device=q.device)
    need = prefill_workspace_size(q, v, N, chunk, emit_every)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = _prefill_args(q, k, v, g, beta, initial_state, final_state, o, cu, N, chunk, scale, l2norm,
                      workspace if need else None, erase, emit_every, chunk_states if emit_every > 0 else None,
                      state_idx, state_dtype)
    _check(lib().gdn_prefill(ctypes.byref(a), _stream(q.device)), "gdn_prefill")
    if emit_every > 0:
        return o, final_state, chunk_states
    return o, final_state


NOALLOC_MAX_SEQS = 8192


def prefill_noalloc(q, k, v, g, beta, initial_state, cu_seqlens, o, final_state, chunk=64, scale=1.0,
                    l2norm=True, erase=True, emit_every=0, chunk_states=None, state_idx=None):
    """gdn_prefill_noalloc: prefill into caller-given outputs (o, final_state
    or None, chunk_states when emit_every > 0) with no workspace and no
    allocation inside the call; bf16 io at chunk 32 or 64, at most
    NOALLOC_MAX_SEQS sequences.  The plan lives in a static per-GPU array:
    calls that overlap on one GPU race."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _head_view(t, nm)
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    cu, N = _cu(cu_seqlens, q.shape[0])
    given = [t for t in (initial_state, final_state, chunk_states) if t is not None]
    state_dtype = given[0].dtype if given else torch.float32
    a = _prefill_args(q, k, v, g, beta, initial_state, final_state, o, cu, N, chunk, scale, l2norm, None, erase,
                      emit_every, chunk_states, state_idx, state_dtype)
    _check(lib().gdn_prefill_noalloc(ctypes.byref(a), _stream(q.device)), "gdn_prefill_noalloc")
    return o, final_state


def split_qkv(y, h_qk, d_k, h_v, d_v):
    """Column views [q | k | v] of the conv output y [T, C] as [T, H, d] tensors."""
    T = y.shape[0]
    nq = h_qk * d_k
    q = y[:, :nq].unflatten(1, (h_qk, d_k))
    k = y[:, nq:2 * nq].unflatten(1, (h_qk, d_k))
    v = y[:, 2 * nq:2 * nq + h_v * d_v].unflatten(1, (h_v, d_v))
    return q, k, v


def gdn_layer(x, conv_weight, g, beta, h_qk, d_k, h_v, d_v, conv_bias=None, conv_state=None,
              initial_state=None, cu_seqlens=None, chunk=64, scale=1.0, l2norm=True, y=None,
              erase=True):
    """The whole mixer: conv1d(+SiLU) over [q|k|v], then the chunked recurrence
    reading q, k, v as column slices of the conv output (no copies)."""
    y = conv1d(x, conv_weight, conv_bias, conv_state, cu_seqlens, "silu", out=y)
    q, k, v = split_qkv(y, h_qk, d_k, h_v, d_v)
    o, S = prefill(q, k, v, g, beta, initial_state, cu_seqlens, chunk, scale, l2norm, erase=erase)
    return o, S


def decode_step(x, g, beta, state, h_qk, h_v, d, conv_weight=None, conv_state=None, conv_bias=None,
                activation="silu", l2norm=True, scale=1.0, o=None, erase=True, state_idx=None,
                conv_head=None):
    """One token for each of N sequences.  x [N, C] (pre-conv, or q|k|v when
    conv_weight is None); state [N, H_v, d, d] (bf16 or fp32) and conv_state
    [N, C, W-1] are updated in place.  Returns o [N, H_v, d].  erase=False runs
    the erase-off variant; state_idx [N] int32 picks each sequence's slot of
    the state and conv_state pools; conv_head (int32, one per conv-state slot)
    makes the conv state a ring: one slot is written and the head advances."""
    _contig(x, "x")
    N = x.shape[0]
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(state, "state")
    if conv_weight is not None:
        _contig(conv_weight, "conv_weight", x.dtype)
        _contig(conv_state, "conv_state", x.dtype)
    if conv_bias is not None:
        _contig(conv_bias, "conv_bias", x.dtype)
    if state_idx is not None:
        _contig(state_idx, "state_idx", torch.int32)
    if conv_head is not None:
        _contig(conv_head, "conv_head", torch.int32)
    if o is None:
        o = torch.empty((N, h_v, d), dtype=x.dtype, device=x.device)
    W = conv_weight.shape[1] if conv_weight is not None else 4
    flags = (FLAG_L2NORM_QK if l2norm else 0) | (0 if erase else FLAG_NO_ERASE)
    a = DecodeArgs(ctypes.sizeof(DecodeArgs), flags, _DT[x.dtype],
                   _DT[state.dtype], N, h_qk, h_v, d, d, W,
                   ACT_SILU if activation == "silu" else ACT_NONE, scale, _ptr(x), _ptr(conv_weight),
                   _ptr(conv_bias), _ptr(conv_state), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                   _ptr(state_idx), _ptr(conv_head))
    _check(lib().gdn_decode_step(ctypes.byref(a), _stream(x.device)), "gdn_decode_step")
    return o


def prefill_backward_workspace_size(q, v, n_seqs=1, chunk=64):
    T, h_qk, d_k = q.shape
    a = PrefillBwdArgs(struct_size=ctypes.sizeof(PrefillBwdArgs), io_dtype=_DT[q.dtype], n_seqs=n_seqs,
                       total_tokens=T, h_qk=h_qk, h_v=v.shape[1], d_k=d_k, d_v=v.shape[2], chunk=chunk)
    return lib().gdn_prefill_backward_workspace_size(ctypes.byref(a))


def prefill_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, cu_seqlens=None, chunk=64,
                     scale=1.0, l2norm=True, erase=True, dq=None, dk=None, dv=None, dg=None, dbeta=None,
                     d_initial_state=True, workspace=None):
    """Gradients of prefill: given its inputs and d_o [T, H_v, d] (io dtype),
    d_final_state [N, H_v, d, d] fp32 or None, returns (dq, dk, dv, dg, dbeta,
    d_initial_state).  dq, dk, dv may be passed as [T, H, d] views (token
    stride free) to write into, e.g. column slices of the conv output's
    gradient; d_initial_state=False skips that output."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _head_view(t, nm)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise GdnError("q, k and v must share a dtype")
    T, h_qk, d = q.shape
    h_v = v.shape[1]
    _contig(g, "g", torch.float32)
    _contig(beta, "beta", torch.float32)
    _contig(d_o, "d_o", q.dtype)
    cu, N = _cu(cu_seqlens, T)
    if initial_state is not None:
        _contig(initial_state, "initial_state", torch.float32)
    if d_final_state is not None:
        _contig(d_final_state, "d_final_state", torch.float32)
    dev = q.device
    dq = torch.empty((T, h_qk, d), dtype=q.dtype, device=dev) if dq is None else _head_view(dq, "dq")
    dk = torch.empty((T, h_qk, d), dtype=q.dtype, device=dev) if dk is None else _head_view(dk, "dk")
    dv = torch.empty((T, h_v, d), dtype=q.dtype, device=dev) if dv is None else _head_view(dv, "dv")
    dg = torch.empty((T, h_v), dtype=torch.float32, device=dev) if dg is None else _contig(dg, "dg", torch.float32)
    dbeta = (torch.empty((T, h_v), dtype=torch.float32, device=dev) if dbeta is None
             else _contig(dbeta, "dbeta", torch.float32))
    if d_initial_state is True:
        d_initial_state = torch.empty((N, h_v, d, d), dtype=torch.float32, device=dev)
    elif d_initial_state is False:
        d_initial_state = None
    need = prefill_backward_workspace_size(q, v, N, chunk)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    flags = (FLAG_L2NORM_QK if l2norm else 0) | (0 if erase else FLAG_NO_ERASE)
    a = PrefillBwdArgs(ctypes.sizeof(PrefillBwdArgs), flags, _DT[q.dtype], N, T, h_qk, h_v, d, d, chunk, scale,
                       _ptr(q), _ptr(k), _ptr(v), q.stride(0), k.stride(0), v.stride(0), _ptr(g), _ptr(beta),
                       _ptr(initial_state), _ptr(cu), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                       _ptr(dv), dq.stride(0), dk.stride(0), dv.stride(0), _ptr(dg), _ptr(dbeta),
                       _ptr(d_initial_state), _ptr(workspace), workspace.numel())
    _check(lib().gdn_prefill_backward(ctypes.byref(a), _stream(dev)), "gdn_prefill_backward")
    return dq, dk, dv, dg, dbeta, d_initial_state


def conv1d_backward_workspace_size(T, C):
    a = ConvBwdArgs(struct_size=ctypes.sizeof(ConvBwdArgs), total_tokens=T, channels=C)
    return lib().gdn_conv1d_backward_workspace_size(ctypes.byref(a))


def conv1d_backward(x, weight, dy, bias=None, conv_state=None, cu_seqlens=None, activation="silu",
                    d_new_state=None, dx=None, d_conv_state=True, workspace=None):
    """Gradients of conv1d: returns (dx [T, C] in x's dtype, dweight [C, W] fp32,
    dbias [C] fp32 or None, d_conv_state [N, C, W-1] fp32 or None).
    conv_state is the state the forward call read (before its update)."""
    _contig(x, "x")
    T, C = x.shape
    _contig(weight, "weight", x.dtype)
    _contig(dy, "dy", x.dtype)
    if bias is not None:
        _contig(bias, "bias", x.dtype)
    if conv_state is not None:
        _contig(conv_state, "conv_state", x.dtype)
    if d_new_state is not None:
        _contig(d_new_state, "d_new_state", torch.float32)
    cu, N = _cu(cu_seqlens, T)
    W = weight.shape[1]
    dev = x.device
    dx = torch.empty_like(x) if dx is None else _contig(dx, "dx", x.dtype)
    dweight = torch.empty((C, W), dtype=torch.float32, device=dev)
    dbias = None if bias is None else torch.empty(C, dtype=torch.float32, device=dev)
    if d_conv_state is True:
        d_conv_state = torch.empty((N, C, W - 1), dtype=torch.float32, device=dev)
    elif d_conv_state is False:
        d_conv_state = None
    need = conv1d_backward_workspace_size(T, C)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    a = ConvBwdArgs(ctypes.sizeof(ConvBwdArgs), _DT[x.dtype], N, C, T, W,
                    ACT_SILU if activation == "silu" else ACT_NONE, _ptr(x), _ptr(weight), _ptr(bias),
                    _ptr(conv_state), _ptr(cu), _ptr(dy), _ptr(d_new_state), _ptr(dx), _ptr(dweight),
                    _ptr(dbias), _ptr(d_conv_state), _ptr(workspace), workspace.numel())
    _check(lib().gdn_conv1d_backward(ctypes.byref(a), _stream(dev)), "gdn_conv1d_backward")
    return dx, dweight, dbias, d_conv_state


def gdn_layer_backward(x, conv_weight, g, beta, h_qk, d_k, h_v, d_v, d_o, conv_bias=None, conv_state=None,
                       initial_state=None, cu_seqlens=None, chunk=64, scale=1.0, l2norm=True, erase=True,
                       d_final_state=None, d_new_conv_state=None, y=None):
    """Gradients of gdn_layer: recomputes the conv output y (unless given),
    runs prefill_backward writing dq, dk, dv straight into the conv output's
    gradient dy [T, C], then conv1d_backward.  conv_state is the state the
    forward read.  Returns (dx, dconv_weight, dconv_bias, dg, dbeta,
    d_initial_state, d_conv_state)."""
    if y is None:
        y = conv1d(x, conv_weight, conv_bias, None if conv_state is None else conv_state.clone(), cu_seqlens,
                   "silu")
    q, k, v = split_qkv(y, h_qk, d_k, h_v, d_v)
    dy = torch.zeros_like(y)
    dq, dk, dv = split_qkv(dy, h_qk, d_k, h_v, d_v)
    _, _, _, dg, dbeta, ds0 = prefill_backward(q, k, v, g, beta, d_o, initial_state, d_final_state, cu_seqlens,
                                               chunk, scale, l2norm, erase, dq=dq, dk=dk, dv=dv)
    dx, dw, db, dcs = conv1d_backward(x, conv_weight, dy, conv_bias, conv_state, cu_seqlens, "silu",
                                      d_new_conv_state)
    return dx, dw, db, dg, dbeta, ds0, dcs


def probe_mfma(iters=2048, blocks=2048, device=None):
    """Measured dense bf16 MFMA rate: one launch of the library's MFMA probe
    (blocks x 4 waves, each iters x 8 independent 16x16x32 MFMAs), timed with
    HIP events on the current stream.  Returns TFLOP/s."""
    dev = device or torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    L = lib()
    st = _stream(dev)
    _check(L.gdn_probe_mfma(iters, blocks, _ptr(out), st), "gdn_probe_mfma")  # warm-up
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    _check(L.gdn_probe_mfma(iters, blocks, _ptr(out), st), "gdn_probe_mfma")
    b.record()
    torch.cuda.synchronize(dev)
    return L.gdn_probe_mfma_flops(iters, blocks) / (a.elapsed_time(b) * 1e-3) / 1e12


def probe_copy(nbytes=1 << 30, reps=5, device=None):
    """Measured streaming copy rate (read + write bytes / s) of a device copy
    of nbytes through the library's copy probe, best of reps.  Returns GB/s."""
    dev = device or torch.device("cuda", torch.cuda.current_device())
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    L = lib()
    st = _stream(dev)
    best = 0.0
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        _check(L.gdn_probe_copy(_ptr(src), _ptr(dst), nbytes, st), "gdn_probe_copy")
        b.record()
        torch.cuda.synchronize(dev)
        best = max(best, 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    return best
