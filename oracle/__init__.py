"""KDA oracle: plain fp64 CPU reference for parity tests.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
package ``kda_gated_delta_chunk_amd`` never imports it, and the two share no
code: the only thing both sides use is the seeded input generator
(``kda_gated_delta_chunk_amd.synth``), which holds none of the method's
arithmetic.

The arithmetic lives in ``kda_oracle.c`` (per-token recurrence, see the
citations there). This module compiles it with gcc and calls it via ctypes.
Every array is widened to float64 before the call, so the oracle sees exactly
the values the GPU received (bf16 or fp32), just held in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "kda_oracle.c"
_LIB = _HERE / "libkda_oracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile the C oracle with gcc (-O2, no fast-math)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build(force=True)
        lib = ctypes.CDLL(str(_LIB))
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.kda_oracle_chunk_fwd.argtypes = [dp, dp, dp, dp, dp, dp, ip,
                                             i64, i64, i64, i64, i64, i64, dp, dp, ctypes.c_int]
        lib.kda_oracle_chunk_fwd.restype = ctypes.c_int
        lib.kda_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, dp,
                                          i64, i64, i64, i64, ctypes.c_int]
        lib.kda_oracle_decode.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Widen to a C-contiguous float64 copy (exact for bf16/fp16/fp32 inputs)."""
    if hasattr(x, "detach"):  # a torch tensor: copy to host, widen exactly
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


GATES = ("log_decay", "scaled_sigmoid")


def scaled_sigmoid_gate(x) -> np.ndarray:
    """Log-decay from the gate pre-activation x, in fp64: -5 * sigmoid(x) = -5 / (1 + e^(-x)).

    "Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
    "K3 对 Kimi Linear 的进一步修改": K3's log-decay is a sigmoid scaled to a
    lower bound of -5 (in place of Kimi Linear's unbounded negative softplus).
    The plainest reading of "scaled sigmoid bounded below by -5" for a
    log-decay (which must be <= 0) is -5 * sigmoid(x), range (-5, 0).
    """
    x = _f64(x)
    with np.errstate(over="ignore"):  # e^(-x) = inf for x < -709: the result is -0 (no decay)
        return -5.0 / (1.0 + np.exp(-x))


def output_gate(o, z) -> np.ndarray:
    """The output gate, in fp64: o * sigmoid(z), channel by channel.

    "Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
    "K3 对 Kimi Linear 的进一步修改": KDA's low-rank output gate became an
    input-dependent, full-rank channel gate, one value per output channel and
    token. The pages name no activation; sigmoid, the plain form of a gate, is
    the reading taken. z is the gate's pre-activation (the projection that
    makes it from the layer input is upstream of this path).
    """
    z = _f64(z)
    with np.errstate(over="ignore"):
        return _f64(o) * (1.0 / (1.0 + np.exp(-z)))


L2NORM_EPS = 1e-6


def l2_normalize(x) -> np.ndarray:
    """Each vector along the last axis divided by its L2 norm, in fp64: x / sqrt(sum(x^2) + eps).

    The pages give KDA's per-channel decay, the delta-rule write and the read
    but say nothing about normalising q and k ("Kimi K3 发布核实与 Moonshot AI
    主干架构演变", section 3, paragraph "KDA 为什么不同于 MLA"). The delta rule
    of "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE", section 二.3
    (read what the key maps to, write back only the error) is an exact
    overwrite only for a unit-norm key, so unit-norm keys (and queries) are
    read as the optional prologue of the path. eps = 1e-6 under the root keeps
    an all-zero vector at zero instead of dividing by zero.
    """
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)


CONVS = ("none", "short4", "short4_silu")


def silu(x) -> np.ndarray:
    """x * sigmoid(x), in fp64."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def short_conv(x, w, seq_start, act: str = "short4") -> np.ndarray:
    """Causal depthwise convolution of length 4 over tokens, in fp64.

    "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE", section 二.3 (last
    paragraph): KDA is combined with a short convolution of length 4 that mixes
    neighbouring tokens. The pages give neither the exact form nor an
    activation; the reading taken is the plain causal depthwise one, each
    channel of each head on its own:
        y_t[h, c] = sum_{j=0..3} w[h, c, j] * x_{t-3+j}[h, c]
    (w[..., 3] weights the current token), where tokens before the start of
    t's sequence count as zero, optionally followed by SiLU (act
    "short4_silu"). x: [T, H, D] of one packed row; w: [H, D, 4];
    seq_start: [T] int, the first token of each token's sequence.
    """
    x = _f64(x)
    w = _f64(w)
    T = x.shape[0]
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(4):
            tau = t - 3 + j
            if tau >= seq_start[t]:
                y[t] += w[:, :, j] * x[tau]
    return silu(y) if act == "short4_silu" else y


def _seq_starts(B, T, cu):
    """First token of each token's sequence, per batch row ([B, T])."""
    st = np.zeros((B, T), dtype=np.int64)
    if cu is None:
        return st
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        st[0, a:b] = a
    return st


def _apply_conv(q, k, v, conv, conv_w, cu):
    """The short convolution of q, k and v (conv_w [H, K + K + V, 4]: q channels, then k, then v)."""
    if conv not in CONVS:
        raise ValueError("conv must be one of %s" % (CONVS,))
    if conv == "none":
        return q, k, v
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, K = q.shape
    V = v.shape[-1]
    w = _f64(conv_w)
    if w.shape != (H, 2 * K + V, 4):
        raise ValueError("conv_w shape %s != %s" % (w.shape, (H, 2 * K + V, 4)))
    st = _seq_starts(B, T, cu)
    out = []
    for x, lo, hi in ((q, 0, K), (k, K, 2 * K), (v, 2 * K, 2 * K + V)):
        out.append(np.stack([short_conv(x[b], w[:, lo:hi], st[b], conv) for b in range(B)]))
    return out


def _log_decay(g, gate: str) -> np.ndarray:
    if gate not in GATES:
        raise ValueError("gate must be one of %s" % (GATES,))
    return scaled_sigmoid_gate(g) if gate == "scaled_sigmoid" else _f64(g)


def chunk_fwd(q, k, v, g, beta, S0=None, cu_seqlens=None, threads: int = 0, gate: str = "log_decay",
              o_gate=None, qk_norm: bool = False, conv: str = "none", conv_w=None):
    """Run the fp64 recurrence over whole sequences.

    q, k, g: [B, T, H, K]; v: [B, T, H, V]; beta: [B, T, H];
    S0: [N, H, K, V] or None (zeros); cu_seqlens: [N+1] or None.
    gate: "log_decay" (g is the log-decay) or "scaled_sigmoid" (g is the gate
    pre-activation; the log-decay is scaled_sigmoid_gate(g)).
    o_gate: [B, T, H, V] or None; if given, o is output_gate(o, o_gate).
    qk_norm: if true, q and k are replaced by l2_normalize(q), l2_normalize(k)
    (per token and head, over the K key channels) before the recurrence.
    conv: "none", "short4" or "short4_silu": q, k and v first go through
    short_conv with the weights conv_w [H, K + K + V, 4] (q channels, then k,
    then v), restarting at every sequence start; the normalisation follows.
    Returns (o [B, T, H, V], S_final [N, H, K, V]) as float64 arrays.
    """
    g = _log_decay(g, gate)
    if conv != "none":
        cu_np = None
        if cu_seqlens is not None:
            cu_np = cu_seqlens.detach().cpu().numpy() if hasattr(cu_seqlens, "detach") else np.asarray(cu_seqlens)
        q, k, v = _apply_conv(q, k, v, conv, conv_w, cu_np)
    if qk_norm:
        q, k = l2_normalize(q), l2_normalize(k)
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, V) or beta.shape != (B, T, H):
        raise ValueError("inconsistent input shapes")
    cu = None
    if cu_seqlens is not None:
        if hasattr(cu_seqlens, "detach"):
            cu_seqlens = cu_seqlens.detach().cpu().numpy()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
    else:
        N = B
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (N, H, K, V):
        raise ValueError("S0 shape %s != %s" % (s0.shape, (N, H, K, V)))
    o = np.zeros((B, T, H, V), dtype=np.float64)
    sf = np.zeros((N, H, K, V), dtype=np.float64)
    cu_ptr = None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    rc = _load().kda_oracle_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), cu_ptr,
                                      B, T, H, K, V, N, _ptr(o), _ptr(sf), int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if o_gate is not None:
        if tuple(o_gate.shape) != o.shape:
            raise ValueError("o_gate shape %s != %s" % (tuple(o_gate.shape), o.shape))
        o = output_gate(o, o_gate)
    return o, sf


def decode_step(q, k, v, g, beta, S, threads: int = 0, gate: str = "log_decay", o_gate=None,
                qk_norm: bool = False, conv: str = "none", conv_w=None, conv_cache=None):
    """One decode step. q, k, g: [N, H, K]; v: [N, H, V]; beta: [N, H]; S: [N, H, K, V].

    gate, o_gate ([N, H, V] or None), qk_norm, conv and conv_w as for chunk_fwd.
    With a conv, conv_cache [N, H, 3, K + K + V] holds the raw q | k | v of the
    three previous tokens of each sequence, oldest first (zeros before the
    sequence start): the token is convolved over those three and itself.
    Returns (o [N, H, V], S_new [N, H, K, V]) and, with a conv, the new cache
    (the last two rows moved up, the raw token appended); the inputs are not
    modified.
    """
    g = _log_decay(g, gate)
    new_cache = None
    if conv != "none":
        if conv not in CONVS:
            raise ValueError("conv must be one of %s" % (CONVS,))
        cache = _f64(conv_cache)
        raw = np.concatenate([_f64(q), _f64(k), _f64(v)], axis=-1)  # [N, H, K + K + V]
        Kq = q.shape[-1]
        win = np.concatenate([cache, raw[:, :, None, :]], axis=2)   # [N, H, 4, K + K + V] oldest first
        y = np.einsum("nhjc,hcj->nhc", win, _f64(conv_w))
        if conv == "short4_silu":
            y = silu(y)
        q, k, v = y[..., :Kq], y[..., Kq:2 * Kq], y[..., 2 * Kq:]
        new_cache = win[:, :, 1:, :].copy()
    if qk_norm:
        q, k = l2_normalize(q), l2_normalize(k)
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    S_new = _f64(S).copy()
    N, H, K = q.shape
    V = v.shape[-1]
    if S_new.shape != (N, H, K, V):
        raise ValueError("state shape mismatch")
    o = np.zeros((N, H, V), dtype=np.float64)
    rc = _load().kda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S_new), _ptr(o),
                                   N, H, K, V, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    if o_gate is not None:
        if tuple(o_gate.shape) != o.shape:
            raise ValueError("o_gate shape %s != %s" % (tuple(o_gate.shape), o.shape))
        o = output_gate(o, o_gate)
    if conv != "none":
        return o, S_new, new_cache
    return o, S_new


def parity_error(x, ref) -> float:
    """max|x - ref| / rms(ref), the comparison metric used by every parity test."""
    x = _f64(x)
    ref = _f64(ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    diff = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if rms == 0.0:
        return diff
    return diff / rms


from .backward import chunk_bwd  # noqa: E402  (gradients of chunk_fwd, fp64 numpy)
