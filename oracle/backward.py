"""Gradients of the KDA recurrence: plain fp64 reverse pass (numpy).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the
smoke check and the benchmark's CPU baseline leg may use it.

What it differentiates is the per-token recurrence of the forward oracle
("Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
"KDA 为什么不同于 MLA": decay per channel, then the delta-rule correction,
then the read of the updated state; the same paragraph names the chunked
form as the way the layer is trained). Per sequence and head, with
S in R^{K x V}:

    A_t = diag(exp(g_t)) S_{t-1}          decayed state
    d_t = v_t - A_t^T k_t                 delta-rule error
    S_t = A_t + beta_t k_t d_t^T          corrected state
    o_t = S_t^T q_t                       read

The pages print no backward pass; the gradients below are the chain rule
applied to those four lines, token by token in reverse order. With
G = dL/dS_t (starting from dL/dS_final, or zero) and do_t = dL/do_t:

    G     += q_t do_t^T                   (o_t reads S_t)
    dq_t   = S_t do_t
    w      = G^T k_t                      (V-vector)
    dv_t   = beta_t w                     (d_t enters S_t as beta k d^T)
    dbeta_t= w . d_t
    dk_t   = beta_t G d_t - A_t dv_t      (k in beta k d^T, and in d = v - A^T k)
    GA     = G - k_t dv_t^T               (dL/dA_t: A_t enters S_t and d_t)
    dg_t   = rowsum(GA * A_t)             (A_t = diag(e^g) S_{t-1}, dA/dg_r = A_t[r, :])
    G      = diag(exp(g_t)) GA            (dL/dS_{t-1})

and dL/dS0 is the final G. With the scaled-sigmoid gate ("Kimi K3 发布核实与 Moonshot AI 主干架构演变",
section 3, paragraph "K3 对 Kimi Linear 的进一步修改": the log-decay is a sigmoid scaled to a lower bound
of -5) g holds the pre-activation x, the log-decay is -5 sigmoid(x), and its gradient is carried to x by
the derivative -5 sigmoid(x) (1 - sigmoid(x)). With the output gate (same paragraph: an input-dependent,
full-rank channel gate on the output, read as o_t * sigmoid(z_t)), the reverse pass takes
do_t * sigmoid(z_t) as the core output's gradient, and dL/dz_t = do_t * o_t * sigmoid(z_t) (1 - sigmoid(z_t))
with o_t = S_t^T q_t the core output. The forward states A_t and d_t are kept from a
plain forward run (no recomputation).

The prologue of the forward oracle (oracle.chunk_fwd) is taken back through the chain rule as well:
- the q/k normalisation x_n = r x with r = (|x|^2 + eps)^(-1/2) ("Kimi K3 模型架构解析：KDA、AttnRes 与
  Stable LatentMoE", section 二.3: the delta rule overwrites exactly for unit-norm keys) has
  dL/dx = r (dL/dx_n - (x_n . dL/dx_n) x_n);
- the short convolution y_t = sum_j w_j x_{t-3+j} over the tokens of t's sequence (same page, last
  paragraph of section 二.3), optionally followed by SiLU z = y sigmoid(y) with dz/dy =
  sigmoid(y) (1 + y (1 - sigmoid(y))), has dL/dx_s = sum_j w_j dL/dy_{s+3-j} over the t = s+3-j of s's
  sequence and dL/dw_j = sum_t dL/dy_t x_{t-3+j} over the pairs inside a sequence.

Parity of this function is pinned against central finite differences of the C forward oracle (through
its own gate, output-gate, normalisation and convolution switches), exact linearity in (v, S0) and in q,
and a closed form at beta = 0, g = 0.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _sequences(B, T, cu):
    """(batch row, first token, end token) of every sequence."""
    if cu is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in cu]
    if B != 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must run from 0 to T, non-decreasing, with B = 1")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def _conv_back(x, w, dz, seq_start, act):
    """The short convolution's reverse for one tensor of one packed row: x [T, H, D] (the convolution's
    input), w [H, D, 4], dz [T, H, D] = dL/d(output), seq_start [T]. Returns (dL/dx, dL/dw)."""
    T = x.shape[0]
    y = np.zeros_like(x)
    for t in range(T):
        for j in range(4):
            tau = t - 3 + j
            if tau >= seq_start[t]:
                y[t] += w[:, :, j] * x[tau]
    if act == "short4_silu":
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-y))
        dy = dz * sg * (1.0 + y * (1.0 - sg))
    else:
        dy = dz
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for t in range(T):
        for j in range(4):
            tau = t - 3 + j
            if tau >= seq_start[t]:
                dx[tau] += w[:, :, j] * dy[t]
                dw[:, :, j] += dy[t] * x[tau]
    return dx, dw


def _norm_back(xn, r, dxn):
    """The reverse of x_n = r x, r = (|x|^2 + eps)^(-1/2), along the last axis: dL/dx from x_n, r and
    dL/dx_n."""
    return r * (dxn - np.sum(xn * dxn, axis=-1, keepdims=True) * xn)


def chunk_bwd(q, k, v, g, beta, do, S0=None, dS_final=None, cu_seqlens=None, gate: str = "log_decay",
              o_gate=None, qk_norm: bool = False, conv: str = "none", conv_w=None):
    """Gradients of (o, S_final) = chunk_fwd(q, k, v, g, beta, S0, cu_seqlens, gate=..., o_gate=...,
    qk_norm=..., conv=..., conv_w=...): with the prologue, q, k and v are the raw inputs the forward
    convolves and normalises, their gradients are taken back through both, and the result also holds
    "dconv_w" [H, K + K + V, 4] (with a convolution).

    q, k, g: [B, T, H, K]; v, do: [B, T, H, V]; beta: [B, T, H];
    S0, dS_final: [N, H, K, V] or None (zeros). gate: "log_decay" (g is the log-decay) or "scaled_sigmoid"
    (g is the gate pre-activation x; the returned dg is then dL/dx). o_gate: the output gate's pre-activation
    z [B, T, H, V] or None; with it, do is the gradient of the gated output and the result also holds
    "do_gate" = dL/dz.
    Returns a dict of float64 arrays: dq, dk, dg [B, T, H, K]; dv [B, T, H, V];
    dbeta [B, T, H]; dS0 [N, H, K, V]. cu_seqlens, if given, runs from 0 to T.
    """
    q, k, v, g, beta, do = (_f64(x) for x in (q, k, v, g, beta, do))
    if gate not in ("log_decay", "scaled_sigmoid"):
        raise ValueError("unknown gate %r" % (gate,))
    if conv not in ("none", "short4", "short4_silu"):
        raise ValueError("unknown conv %r" % (conv,))
    if cu_seqlens is not None and hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    # the prologue, forward: convolution (with SiLU), then the q/k normalisation
    q_raw, k_raw, v_raw = q, k, v
    if conv != "none":
        from . import _apply_conv
        q, k, v = _apply_conv(q, k, v, conv, conv_w, cu_seqlens)
    q_c, k_c = q, k
    rq = rk = None
    if qk_norm:
        from . import L2NORM_EPS
        rq = 1.0 / np.sqrt(np.sum(q_c * q_c, axis=-1, keepdims=True) + L2NORM_EPS)
        rk = 1.0 / np.sqrt(np.sum(k_c * k_c, axis=-1, keepdims=True) + L2NORM_EPS)
        q, k = q_c * rq, k_c * rk
    x_pre = None
    if gate == "scaled_sigmoid":
        from . import scaled_sigmoid_gate
        x_pre, g = g, scaled_sigmoid_gate(g)
    B, T, H, K = q.shape
    V = v.shape[-1]
    z = None if o_gate is None else _f64(o_gate)
    if z is not None:
        if z.shape != (B, T, H, V):
            raise ValueError("o_gate shape %s != %s" % (z.shape, (B, T, H, V)))
        sz = 1.0 / (1.0 + np.exp(-z))
        do_raw, do = do, do * sz
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, V) or do.shape != v.shape \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent input shapes")
    seqs = _sequences(B, T, cu_seqlens)
    N = len(seqs)
    s0 = None if S0 is None else _f64(S0)
    dsf = None if dS_final is None else _f64(dS_final)
    for x in (s0, dsf):
        if x is not None and x.shape != (N, H, K, V):
            raise ValueError("state shape %s != %s" % (x.shape, (N, H, K, V)))
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dg": np.zeros_like(g), "dv": np.zeros_like(v),
           "dbeta": np.zeros_like(beta), "dS0": np.zeros((N, H, K, V))}
    if z is not None:
        out["do_gate"] = np.zeros_like(v)
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((K, V)) if s0 is None else s0[n, h].copy()
            A_hist, d_hist = [], []
            for t in range(t0, t1):                      # forward, keeping A_t and d_t
                A = np.exp(g[b, t, h])[:, None] * S
                d = v[b, t, h] - A.T @ k[b, t, h]
                S = A + beta[b, t, h] * np.outer(k[b, t, h], d)
                A_hist.append(A)
                d_hist.append(d)
            G = np.zeros((K, V)) if dsf is None else dsf[n, h].copy()
            for t in range(t1 - 1, t0 - 1, -1):          # reverse
                A, d = A_hist[t - t0], d_hist[t - t0]
                kt, qt, bt, dot = k[b, t, h], q[b, t, h], beta[b, t, h], do[b, t, h]
                St = A + bt * np.outer(kt, d)
                if z is not None:
                    s_ = sz[b, t, h]
                    out["do_gate"][b, t, h] = do_raw[b, t, h] * (St.T @ qt) * s_ * (1.0 - s_)
                G = G + np.outer(qt, dot)
                out["dq"][b, t, h] = St @ dot
                w = G.T @ kt
                dv = bt * w
                out["dv"][b, t, h] = dv
                out["dbeta"][b, t, h] = w @ d
                out["dk"][b, t, h] = bt * (G @ d) - A @ dv
                GA = G - np.outer(kt, dv)
                out["dg"][b, t, h] = np.sum(GA * A, axis=1)
                G = np.exp(g[b, t, h])[:, None] * GA
            out["dS0"][n, h] = G
    if x_pre is not None:
        sx = 1.0 / (1.0 + np.exp(-x_pre))
        out["dg"] = out["dg"] * (-5.0 * sx * (1.0 - sx))
    # the prologue, reverse: normalisation, then convolution
    if qk_norm:
        for name, xn, r in (("dq", q, rq), ("dk", k, rk)):
            out[name] = _norm_back(xn, r, out[name])
    if conv != "none":
        from . import _seq_starts
        w = _f64(conv_w)
        st = _seq_starts(B, T, cu_seqlens)
        dw = np.zeros_like(w)
        for name, x, lo, hi in (("dq", q_raw, 0, K), ("dk", k_raw, K, 2 * K), ("dv", v_raw, 2 * K, 2 * K + V)):
            dx = np.zeros_like(x)
            for b in range(B):
                dx[b], dwb = _conv_back(x[b], w[:, lo:hi], out[name][b], st[b], conv)
                dw[:, lo:hi] += dwb
            out[name] = dx
        out["dconv_w"] = dw
    return out
