"""MI355X (gfx950) Kimi Delta Attention hot path: chunked prefill and decode.

The compute lives in libkda.so (hand-written HIP kernels behind the C ABI of
include/kda.h). This module marshals torch tensors into that ABI: it checks
shapes, dtypes and devices, allocates the outputs and the workspace with
torch, and passes raw device pointers plus torch's current HIP stream. It
performs no arithmetic of the method itself.

Shapes (contiguous): q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H];
states [num_seqs, H, K, V] fp32. With cu_seqlens (int32 [num_seqs+1], on the
device), B must be 1 and sequences are packed along T.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import KDAError, KDA_DTYPE_BF16, KDA_DTYPE_FP32

__all__ = ["chunk_fwd", "chunk_prep", "chunk_state", "chunk_bwd", "decode_step", "workspace_bytes",
           "min_workspace_bytes", "prep_workspace_bytes", "workspace_status", "bwd_workspace_bytes", "KDAError",
           "abi_version"]

_DT = {torch.bfloat16: KDA_DTYPE_BF16, torch.float32: KDA_DTYPE_FP32}
_NAME = {"bf16": torch.bfloat16, "fp32": torch.float32}


def abi_version() -> int:
    return _lib.load().kda_abi_version()


def _io_code(dtype) -> int:
    if isinstance(dtype, str):
        dtype = _NAME[dtype]
    if dtype not in _DT:
        raise TypeError("unsupported dtype %s (bf16 or fp32)" % dtype)
    return _DT[dtype]


def _operands_code(operands: str) -> int:
    if operands not in _lib.OPERANDS:
        raise ValueError("operands must be one of %s" % sorted(_lib.OPERANDS))
    return _lib.OPERANDS[operands]


def workspace_bytes(B: int, T: int, H: int, K: int, V: int, num_seqs: int, chunk: int = 16, io="bf16",
                    conv: str = "none", operands: str = "bf16") -> int:
    """Device workspace bytes kda_chunk_fwd needs (0 = unsupported sizes or options)."""
    if conv not in _lib.CONVS:
        raise ValueError("conv must be one of %s" % sorted(_lib.CONVS))
    return int(_lib.load().kda_chunk_fwd_workspace_bytes(B, T, H, K, V, num_seqs, chunk, _io_code(io),
                                                         _lib.CONVS[conv], _operands_code(operands)))


def min_workspace_bytes(B: int, T: int, H: int, K: int, V: int, num_seqs: int, chunk: int = 16, io="bf16",
                        conv: str = "none", operands: str = "bf16") -> int:
    """The least workspace kda_chunk_fwd accepts (below workspace_bytes() it runs the fused low-memory
    form where one exists; 0 = unsupported)."""
    if conv not in _lib.CONVS:
        raise ValueError("conv must be one of %s" % sorted(_lib.CONVS))
    return int(_lib.load().kda_chunk_fwd_min_workspace_bytes(B, T, H, K, V, num_seqs, chunk, _io_code(io),
                                                             _lib.CONVS[conv], _operands_code(operands)))


def prep_workspace_bytes(B: int, T: int, H: int, K: int, V: int, num_seqs: int, chunk: int = 16, io="bf16",
                         conv: str = "none", operands: str = "bf16") -> int:
    """Device workspace bytes a kda_chunk_prep / kda_chunk_state pair needs (0 = unsupported)."""
    if conv not in _lib.CONVS:
        raise ValueError("conv must be one of %s" % sorted(_lib.CONVS))
    return int(_lib.load().kda_chunk_prep_workspace_bytes(B, T, H, K, V, num_seqs, chunk, _io_code(io),
                                                          _lib.CONVS[conv], _operands_code(operands)))


def workspace_status(workspace, stream=None) -> int:
    """Device-side error bits recorded in a prefill workspace (0 = none; _lib.WS_ERR_*). Synchronises
    the stream (default: torch's current stream on the workspace's device)."""
    import ctypes
    lib = _lib.load()
    dev = workspace.device
    sh = _stream(dev) if stream is None else stream
    out = ctypes.c_int32(-1)
    _lib.check(lib.kda_workspace_status(_ptr(workspace), workspace.numel(), ctypes.byref(out), sh),
               "kda_workspace_status")
    return int(out.value)


def bwd_workspace_bytes(B: int, T: int, H: int, K: int, V: int, num_seqs: int, qk_norm: bool = False,
                        conv: str = "none") -> int:
    """Device workspace bytes kda_chunk_bwd needs in one call (0 = unsupported sizes)."""
    if conv not in _lib.CONVS:
        raise ValueError("conv must be one of %s" % sorted(_lib.CONVS))
    return int(_lib.load().kda_chunk_bwd_workspace_bytes(B, T, H, K, V, num_seqs, int(bool(qk_norm)),
                                                         _lib.CONVS[conv]))


def bwd_segmented_workspace_bytes(B: int, T: int, H: int, K: int, V: int, num_seqs: int, segment_tokens: int,
                                  qk_norm: bool = False) -> int:
    """Device workspace bytes kda_chunk_bwd needs when it takes the input in segments of segment_tokens
    tokens (a multiple of 32; no convolution); 0 = unsupported."""
    return int(_lib.load().kda_chunk_bwd_segmented_workspace_bytes(B, T, H, K, V, num_seqs, int(bool(qk_norm)), 0,
                                                                   segment_tokens))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, name, shape, dtype, dev):
    if t.device != dev:
        raise ValueError("%s must be on %s" % (name, dev))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _gate_code(gate: str) -> int:
    if gate not in _lib.GATES:
        raise ValueError("gate must be one of %s" % sorted(_lib.GATES))
    return _lib.GATES[gate]


def _qk_code(qk_norm: bool) -> int:
    return _lib.KDA_QK_L2NORM if qk_norm else _lib.KDA_QK_AS_GIVEN


def _conv_code(conv: str, conv_w, H: int, C: int, dev) -> int:
    if conv not in _lib.CONVS:
        raise ValueError("conv must be one of %s" % sorted(_lib.CONVS))
    if conv != "none":
        _need(conv_w, "conv_w", (H, C, 4), torch.float32, dev)
    return _lib.CONVS[conv]


def chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, chunk: int = 16, o_dtype=None,
              output_final_state: bool = True, workspace=None, out=None, gate: str = "log_decay", o_gate=None,
              qk_norm: bool = False, conv: str = "none", conv_w=None, operands: str = "bf16", final_state_out=None,
              low_memory: bool = False):
    """Chunked KDA prefill. Returns (o, S_final or None).

    o is in ``o_dtype`` (default: the input dtype); S_final is fp32
    [num_seqs, H, K, V]. ``workspace`` (uint8 CUDA tensor), ``out`` and
    ``final_state_out`` may be passed to avoid allocations. ``gate`` says what ``g`` holds: "log_decay"
    (the log-decay itself) or "scaled_sigmoid" (the gate pre-activation,
    mapped to -5*sigmoid(g) inside the kernels). ``o_gate`` [B, T, H, V] (input
    dtype), if given, scales the output channel by channel: o * sigmoid(o_gate).
    ``qk_norm``: if true the kernels divide each q and k row (per token and
    head) by sqrt(|x|^2 + 1e-6) as they read it. ``conv``: "none", "short4" or
    "short4_silu": the causal length-4 convolution of q, k and v with the taps
    ``conv_w`` (fp32 [H, K + K + V, 4]), ahead of the normalisation.
    ``operands``: "bf16" (hi + lo bf16 operand pairs, bf16's range) or "fp16"
    (faster; |v| and the state must stay well inside fp16's range).
    ``low_memory``: allocate only the least workspace the call accepts, so that
    it runs as one fused kernel where one exists (no per-chunk factors in memory;
    slower). A ``workspace`` passed in decides the same way by its size.
    """
    lib = _lib.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be CUDA (HIP) tensors")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    io = _io_code(dt)
    gc = _gate_code(gate)
    for name, t, shp in (("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)), ("v", v, (B, T, H, V)),
                         ("beta", beta, (B, T, H))):
        _need(t, name, shp, dt, dev)
    if o_gate is not None:
        _need(o_gate, "o_gate", (B, T, H, V), dt, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    _need(q, "q", (B, T, H, K), dt, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, K, V), torch.float32, dev)
    odt = dt if o_dtype is None else (_NAME[o_dtype] if isinstance(o_dtype, str) else o_dtype)
    if out is None:
        out = torch.empty((B, T, H, V), dtype=odt, device=dev)
    else:
        _need(out, "out", (B, T, H, V), odt, dev)
    S_final = None
    if final_state_out is not None:
        _need(final_state_out, "final_state_out", (N, H, K, V), torch.float32, dev)
        S_final = final_state_out
    elif output_final_state:
        S_final = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    cc = _conv_code(conv, conv_w, H, 2 * K + V, dev)
    oc = _operands_code(operands)
    query = lib.kda_chunk_fwd_min_workspace_bytes if low_memory else lib.kda_chunk_fwd_workspace_bytes
    need = query(B, T, H, K, V, N, chunk, io, cc, oc)
    if need == 0:
        raise KDAError(2, "kda_chunk_fwd_workspace_bytes(B=%d,T=%d,H=%d,K=%d,V=%d,N=%d,chunk=%d,operands=%s)"
                       % (B, T, H, K, V, N, chunk, operands))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    status = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o_gate), _ptr(S0),
                               _ptr(cu_seqlens),
                               B, T, H, K, V, N, chunk, io, gc, _qk_code(qk_norm), cc, _ptr(conv_w), oc,
                               _io_code(odt), _ptr(out), _ptr(S_final),
                               _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(status, "kda_chunk_fwd")
    return out, S_final


def chunk_prep(q, k, g, beta, workspace, cu_seqlens=None, V: int = None, chunk: int = 16, gate: str = "log_decay",
               qk_norm: bool = False, conv: str = "none", conv_w=None, operands: str = "bf16"):
    """The state-independent half of chunk_fwd (kda_chunk_prep): fills ``workspace`` (uint8 CUDA tensor of
    at least prep_workspace_bytes()) with the chunk factors in the ``operands`` format. ``V`` is the value
    width of the chunk_state call that follows (default K)."""
    lib = _lib.load()
    dev = q.device
    B, T, H, K = q.shape
    V = K if V is None else V
    dt = q.dtype
    io = _io_code(dt)
    for name, t, shp in (("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)), ("beta", beta, (B, T, H))):
        _need(t, name, shp, dt, dev)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    cc = _conv_code(conv, conv_w, H, 2 * K + V, dev)
    st = lib.kda_chunk_prep(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), B, T, H, K, V, N, chunk, io,
                            _gate_code(gate), _qk_code(qk_norm), cc, _ptr(conv_w), _operands_code(operands),
                            _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st, "kda_chunk_prep")


def chunk_state(v, workspace, K: int, S0=None, cu_seqlens=None, chunk: int = 16, o_dtype=None, out=None,
                output_final_state: bool = True, o_gate=None, conv: str = "none", conv_w=None, final_state_out=None):
    """The sequential half of chunk_fwd (kda_chunk_state) over a workspace chunk_prep filled; the operand
    format comes from the workspace. Returns (o, S_final or None)."""
    lib = _lib.load()
    dev = v.device
    B, T, H, V = v.shape
    dt = v.dtype
    io = _io_code(dt)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o_gate is not None:
        _need(o_gate, "o_gate", (B, T, H, V), dt, dev)
    if S0 is not None:
        _need(S0, "S0", (N, H, K, V), torch.float32, dev)
    odt = dt if o_dtype is None else (_NAME[o_dtype] if isinstance(o_dtype, str) else o_dtype)
    if out is None:
        out = torch.empty((B, T, H, V), dtype=odt, device=dev)
    else:
        _need(out, "out", (B, T, H, V), odt, dev)
    S_final = None
    if final_state_out is not None:
        _need(final_state_out, "final_state_out", (N, H, K, V), torch.float32, dev)
        S_final = final_state_out
    elif output_final_state:
        S_final = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    cc = _conv_code(conv, conv_w, H, 2 * K + V, dev)
    st = lib.kda_chunk_state(_ptr(v), _ptr(o_gate), _ptr(S0), _ptr(cu_seqlens), B, T, H, K, V, N, chunk, io, cc,
                             _ptr(conv_w), _io_code(odt), _ptr(out), _ptr(S_final), _ptr(workspace),
                             workspace.numel(), _stream(dev))
    _lib.check(st, "kda_chunk_state")
    return out, S_final


def decode_step(q, k, v, g, beta, S, o_dtype=None, out=None, gate: str = "log_decay", o_gate=None,
                qk_norm: bool = False, conv: str = "none", conv_w=None, conv_cache=None):
    """One decode step; S [N, H, K, V] fp32 is updated in place. Returns o [N, H, V].

    ``gate``, ``o_gate`` ([N, H, V]), ``qk_norm``, ``conv`` and ``conv_w`` as for
    :func:`chunk_fwd`. With a convolution, ``conv_cache`` [N, H, 3, K + K + V]
    (input dtype) holds the raw q | k | v of the three previous tokens, oldest
    first; it is updated in place.
    """
    lib = _lib.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be CUDA (HIP) tensors")
    N, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    io = _io_code(dt)
    gc = _gate_code(gate)
    for name, t, shp in (("k", k, (N, H, K)), ("g", g, (N, H, K)), ("v", v, (N, H, V)), ("beta", beta, (N, H))):
        _need(t, name, shp, dt, dev)
    _need(S, "S", (N, H, K, V), torch.float32, dev)
    if o_gate is not None:
        _need(o_gate, "o_gate", (N, H, V), dt, dev)
    odt = dt if o_dtype is None else (_NAME[o_dtype] if isinstance(o_dtype, str) else o_dtype)
    if out is None:
        out = torch.empty((N, H, V), dtype=odt, device=dev)
    else:
        _need(out, "out", (N, H, V), odt, dev)
    cc = _conv_code(conv, conv_w, H, 2 * K + V, dev)
    if cc:
        _need(conv_cache, "conv_cache", (N, H, 3, 2 * K + V), dt, dev)
    status = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o_gate), _ptr(S), _ptr(out),
                                 N, H, K, V, io, gc, _qk_code(qk_norm), cc, _ptr(conv_w) if cc else None,
                                 _ptr(conv_cache) if cc else None, _io_code(odt), _stream(dev))
    _lib.check(status, "kda_decode_step")
    return out


def chunk_bwd(q, k, v, g, beta, do, S0=None, dS_final=None, cu_seqlens=None, want_dS0: bool = True,
              workspace=None, gate: str = "log_decay", o_gate=None, qk_norm: bool = False, conv: str = "none",
              conv_w=None, out=None, segment_tokens: int = 0):
    """Gradients of chunk_fwd's (o, S_final) given dL/do and dL/dS_final, with respect to the raw inputs.
    ``gate``, ``qk_norm``, ``conv`` and ``conv_w`` say what the forward did, as for chunk_fwd; dg is the
    gradient with respect to g as given (the log-decay, or the gate pre-activation). With ``o_gate`` (the
    forward's output-gate pre-activation z), ``do`` is the gradient of the gated output and the result also
    holds ``do_gate`` = dL/dz [B, T, H, V] fp32. With a convolution the result also holds ``dconv_w``
    [H, K + K + V, 4] fp32.

    ``do`` has o's shape and the input dtype; ``dS_final`` is fp32 [num_seqs, H, K, V] or None (zero).
    Returns a dict of fp32 tensors: dq, dk, dg [B, T, H, K]; dv [B, T, H, V]; dbeta [B, T, H]; and
    dS0 [num_seqs, H, K, V] when ``want_dS0``. ``workspace`` (uint8 CUDA tensor) may be passed to avoid
    the allocation, and ``out`` (a dict with some of the result's keys) preallocated fp32 result tensors.
    """
    lib = _lib.load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be CUDA (HIP) tensors")
    B, T, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    io = _io_code(dt)
    gc = _gate_code(gate)
    qc = _qk_code(qk_norm)
    cc = _conv_code(conv, conv_w, H, 2 * K + V, dev)
    for name, t, shp in (("q", q, (B, T, H, K)), ("k", k, (B, T, H, K)), ("g", g, (B, T, H, K)),
                         ("v", v, (B, T, H, V)), ("beta", beta, (B, T, H)), ("do", do, (B, T, H, V))):
        _need(t, name, shp, dt, dev)
    if o_gate is not None:
        _need(o_gate, "o_gate", (B, T, H, V), dt, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None:
            _need(t, name, (N, H, K, V), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dq": (B, T, H, K), "dk": (B, T, H, K), "dg": (B, T, H, K), "dv": (B, T, H, V), "dbeta": (B, T, H)}
    if want_dS0:
        shapes["dS0"] = (N, H, K, V)
    if o_gate is not None:
        shapes["do_gate"] = (B, T, H, V)
    if cc != 0:
        shapes["dconv_w"] = (H, 2 * K + V, 4)
    given = dict(out or {})
    for name in given:
        if name not in shapes:
            raise ValueError("out[%r]: not a result of this call" % (name,))
        _need(given[name], "out[%r]" % (name,), shapes[name], torch.float32, dev)
    out = {name: given.get(name) if name in given else torch.empty(shp, **f32) for name, shp in shapes.items()}
    if segment_tokens:
        need = int(lib.kda_chunk_bwd_segmented_workspace_bytes(B, T, H, K, V, N, qc, cc, segment_tokens))
        if need == 0:
            raise KDAError(2, "kda_chunk_bwd_segmented_workspace_bytes")
    else:
        need = int(lib.kda_chunk_bwd_workspace_bytes(B, T, H, K, V, N, qc, cc))
        if need == 0:
            raise KDAError(2, "kda_chunk_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o_gate), _ptr(S0), _ptr(cu_seqlens),
                           _ptr(do), _ptr(dS_final), B, T, H, K, V, N, io, gc, qc, cc,
                           _ptr(conv_w if cc != 0 else None), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                           _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out.get("do_gate")), _ptr(out.get("dconv_w")),
                           _ptr(out.get("dS0")), _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st, "kda_chunk_bwd")
    return out
