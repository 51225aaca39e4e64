"""Pins of the fp64 backward oracle (oracle.chunk_bwd), independent of its own derivation.

- central finite differences of the C forward oracle (every input entry, tiny sizes);
- exact linearity: (o, S_final) is linear in (v, S0) jointly and o is linear in q, so the change of the
  loss under any perturbation of those equals the inner product with the gradient;
- closed form at beta = 0, g = 0, where S_t = S0 for every t.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, H, K, V, N=None, s0=True):
    N = B if N is None else N
    x = {
        "q": rng.standard_normal((B, T, H, K)),
        "k": rng.standard_normal((B, T, H, K)) * 0.5,
        "v": rng.standard_normal((B, T, H, V)),
        "g": -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, K)))),
        "beta": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
        "S0": rng.standard_normal((N, H, K, V)) * 0.3 if s0 else None,
    }
    do = rng.standard_normal((B, T, H, V))
    dsf = rng.standard_normal((N, H, K, V))
    return x, do, dsf


def _loss(x, do, dsf, cu):
    o, sf = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], cu)
    return float(np.sum(o * do) + np.sum(sf * dsf))


CASES = [
    # (B, T, H, K, V, cu_seqlens)
    (1, 7, 2, 4, 3, None),
    (2, 5, 1, 3, 4, None),
    (1, 9, 2, 3, 2, [0, 3, 3, 9]),      # an empty sequence
    (1, 8, 1, 3, 3, [0, 1, 4, 8]),      # a one-token sequence
]


@pytest.mark.parametrize("case", CASES)
def test_bwd_matches_finite_differences(case):
    B, T, H, K, V, cu = case
    rng = np.random.default_rng(11)
    N = B if cu is None else len(cu) - 1
    x, do, dsf = _inputs(rng, B, T, H, K, V, N)
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, cu)
    eps = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(x, do, dsf, cu)
            flat[i] = old - eps
            lm = _loss(x, do, dsf, cu)
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(fd - gr[gname])) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_bwd_rejects_a_table_that_does_not_cover_the_batch():
    rng = np.random.default_rng(3)
    x, do, dsf = _inputs(rng, 1, 8, 2, 3, 3, 2)
    for cu in ([1, 4, 8], [0, 4, 6], [0, 5, 4]):
        with pytest.raises(ValueError):
            oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, cu)


def test_bwd_exact_linearity_in_v_S0_and_q():
    rng = np.random.default_rng(5)
    B, T, H, K, V = 1, 24, 2, 6, 5
    x, do, dsf = _inputs(rng, B, T, H, K, V)
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf)
    l0 = _loss(x, do, dsf, None)
    dv, ds0, dq = (rng.standard_normal(x[n].shape) for n in ("v", "S0", "q"))
    y = dict(x, v=x["v"] + dv, S0=x["S0"] + ds0)
    pred = np.sum(gr["dv"] * dv) + np.sum(gr["dS0"] * ds0)
    assert abs(_loss(y, do, dsf, None) - l0 - pred) <= 1e-11 * max(1.0, abs(pred))
    y = dict(x, q=x["q"] + dq)
    pred = np.sum(gr["dq"] * dq)
    assert abs(_loss(y, do, dsf, None) - l0 - pred) <= 1e-11 * max(1.0, abs(pred))


def test_bwd_closed_form_no_write_no_decay():
    # beta = 0, g = 0: S_t = S0 for all t and o_t = S0^T q_t. With G_t = dS_final + sum_{s >= t} q_s do_s^T:
    # dq_t = S0 do_t, dk = dv = 0, dbeta_t = (G_t^T k_t) . (v_t - S0^T k_t), dg_t = rowsum(G_t * S0),
    # dS0 = G_1.
    rng = np.random.default_rng(9)
    T, H, K, V = 10, 2, 4, 3
    x, do, dsf = _inputs(rng, 1, T, H, K, V)
    x["beta"][:] = 0.0
    x["g"][:] = 0.0
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf)
    for h in range(H):
        S0 = x["S0"][0, h]
        outer = np.einsum("tk,tv->tkv", x["q"][0, :, h], do[0, :, h])
        G = dsf[0, h][None] + np.cumsum(outer[::-1], axis=0)[::-1]        # G_t for t = 0..T-1
        np.testing.assert_allclose(gr["dq"][0, :, h], do[0, :, h] @ S0.T, rtol=0, atol=1e-13)
        assert np.all(gr["dk"][0, :, h] == 0.0) and np.all(gr["dv"][0, :, h] == 0.0)
        err = x["v"][0, :, h] - x["k"][0, :, h] @ S0
        dbeta = np.einsum("tkv,tk,tv->t", G, x["k"][0, :, h], err)
        np.testing.assert_allclose(gr["dbeta"][0, :, h], dbeta, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gr["dg"][0, :, h], np.sum(G * S0[None], axis=2), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gr["dS0"][0, h], G[0], rtol=1e-12, atol=1e-12)


def _planted(kind):
    """oracle.chunk_bwd with one plausible mistake planted in its reverse step (CPU only)."""
    import oracle.backward as ob

    def bwd(q, k, v, g, beta, do, S0=None, dS_final=None, cu_seqlens=None):
        q, k, v, g, beta, do = (ob._f64(x) for x in (q, k, v, g, beta, do))
        B, T, H, K = q.shape
        V = v.shape[-1]
        out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dg": np.zeros_like(g), "dv": np.zeros_like(v),
               "dbeta": np.zeros_like(beta), "dS0": np.zeros((B, H, K, V))}
        for b in range(B):
            for h in range(H):
                S = ob._f64(S0)[b, h].copy()
                As, ds = [], []
                for t in range(T):
                    A = np.exp(g[b, t, h])[:, None] * S
                    d = v[b, t, h] - A.T @ k[b, t, h]
                    S = A + beta[b, t, h] * np.outer(k[b, t, h], d)
                    As.append(A)
                    ds.append(d)
                G = ob._f64(dS_final)[b, h].copy()
                for t in range(T - 1, -1, -1):
                    A, d, kt, qt, bt, dot = As[t], ds[t], k[b, t, h], q[b, t, h], beta[b, t, h], do[b, t, h]
                    St = A + bt * np.outer(kt, d)
                    if kind != "qdo_late":
                        G = G + np.outer(qt, dot)
                    out["dq"][b, t, h] = (A if kind == "dq_old_state" else St) @ dot
                    w = G.T @ kt
                    dv = bt * w
                    out["dv"][b, t, h] = dv
                    out["dbeta"][b, t, h] = w @ (v[b, t, h] if kind == "dbeta_uses_v" else d)
                    dk = bt * (G @ d) - (0 if kind == "dk_drops_read" else A @ dv)
                    out["dk"][b, t, h] = -dk if kind == "dk_sign" else dk
                    GA = G - (0 if kind == "GA_drops_write" else np.outer(kt, dv))
                    out["dg"][b, t, h] = np.sum((G if kind == "dg_uses_G" else GA) * A, axis=1)
                    G = (GA if kind == "no_decay" else np.exp(g[b, t, h])[:, None] * GA)
                    if kind == "qdo_late":  # q_t do_t^T added after the step's own transform
                        G = G + np.outer(qt, dot)
                out["dS0"][b, h] = G
        return out
    return bwd


@pytest.mark.parametrize("kind", ["dq_old_state", "qdo_late", "dbeta_uses_v", "dk_drops_read", "dk_sign",
                                  "GA_drops_write", "dg_uses_G", "no_decay"])
def test_planted_backward_mistakes_fail_the_finite_difference_pin(kind):
    # each mistake must move at least one gradient well away from the central differences of the C forward
    rng = np.random.default_rng(21)
    B, T, H, K, V = 1, 6, 1, 3, 2
    x, do, dsf = _inputs(rng, B, T, H, K, V)
    ok = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf)
    bad = _planted(kind)(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    worst = 0.0
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 1e-6
            lp = _loss(x, do, dsf, None)
            flat[i] = old - 1e-6
            lm = _loss(x, do, dsf, None)
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / 2e-6
        assert np.max(np.abs(fd - ok[gname])) < 1e-6 * max(1.0, np.max(np.abs(fd)))
        worst = max(worst, np.max(np.abs(fd - bad[gname])) / max(1.0, np.max(np.abs(fd))))
    assert worst > 1e-3, (kind, worst)


def test_bwd_gate_preactivation_matches_finite_differences():
    # g holds the gate pre-activation x (log-decay -5 sigmoid(x)); dg must be dL/dx of the forward oracle run
    # with the same gate switch
    rng = np.random.default_rng(31)
    B, T, H, K, V = 1, 7, 2, 3, 2
    x, do, dsf = _inputs(rng, B, T, H, K, V)
    x["g"] = 2.0 * rng.standard_normal((B, T, H, K))
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, gate="scaled_sigmoid")

    def loss():
        o, sf = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], gate="scaled_sigmoid")
        return float(np.sum(o * do) + np.sum(sf * dsf))
    fd = np.zeros_like(x["g"])
    flat = x["g"].reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + 1e-6
        lp = loss()
        flat[i] = old - 1e-6
        lm = loss()
        flat[i] = old
        fd.reshape(-1)[i] = (lp - lm) / 2e-6
    assert np.max(np.abs(fd - gr["dg"])) < 1e-7 * max(1.0, np.max(np.abs(fd)))
    # the other gradients are those of the log-decay form at g = -5 sigmoid(x)
    ref = oracle.chunk_bwd(x["q"], x["k"], x["v"], oracle.scaled_sigmoid_gate(x["g"]), x["beta"], do, x["S0"], dsf)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.array_equal(gr[n], ref[n]), n


def test_bwd_output_gate_matches_finite_differences():
    # o = core output * sigmoid(z): dL/dz, and the other gradients taken through the gate, against central
    # differences of the forward oracle run with the same output gate
    rng = np.random.default_rng(41)
    B, T, H, K, V = 1, 6, 2, 3, 3
    x, do, dsf = _inputs(rng, B, T, H, K, V)
    x["z"] = rng.standard_normal((B, T, H, V))
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, o_gate=x["z"])

    def loss():
        o, sf = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], o_gate=x["z"])
        return float(np.sum(o * do) + np.sum(sf * dsf))
    for name, gname in (("z", "do_gate"), ("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                        ("S0", "dS0")):
        fd = np.zeros_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 1e-6
            lp = loss()
            flat[i] = old - 1e-6
            lm = loss()
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / 2e-6
        assert np.max(np.abs(fd - gr[gname])) < 1e-7 * max(1.0, np.max(np.abs(fd))), name


PROLOGUE_CASES = [
    # (qk_norm, conv, cu_seqlens): the normalisation alone, each convolution with and without it, packed
    # sequences (an empty and a one-token one) so that the history restarts inside the row
    (True, "none", None),
    (False, "short4", None),
    (True, "short4_silu", None),
    (True, "short4_silu", [0, 4, 4, 5, 9]),
    (False, "short4", [0, 2, 9]),
]


@pytest.mark.parametrize("qk_norm,conv,cu", PROLOGUE_CASES)
def test_bwd_prologue_matches_finite_differences(qk_norm, conv, cu):
    # raw q, k, v go through the short convolution and the normalisation inside the forward oracle: the
    # gradients of every raw input, of the taps and of the other inputs against central differences of the
    # forward oracle run with the same switches (both gates on, so every path of the prologue is taken)
    rng = np.random.default_rng(51)
    B, T, H, K, V = 1, 9, 2, 3, 2
    N = B if cu is None else len(cu) - 1
    x, do, dsf = _inputs(rng, B, T, H, K, V, N)
    x["q"] = rng.standard_normal((B, T, H, K))
    x["k"] = rng.standard_normal((B, T, H, K))
    x["g"] = 2.0 * rng.standard_normal((B, T, H, K))
    x["z"] = rng.standard_normal((B, T, H, V))
    x["w"] = 0.7 * rng.standard_normal((H, 2 * K + V, 4))
    cw = x["w"] if conv != "none" else None
    kw = dict(gate="scaled_sigmoid", o_gate=x["z"], qk_norm=qk_norm, conv=conv, conv_w=cw)
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, cu, **kw)

    def loss():
        o, sf = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], cu, **kw)
        return float(np.sum(o * do) + np.sum(sf * dsf))
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("S0", "dS0"), ("z", "do_gate")]
    if conv != "none":
        names.append(("w", "dconv_w"))
    else:
        assert "dconv_w" not in gr
    for name, gname in names:
        fd = np.zeros_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 1e-6
            lp = loss()
            flat[i] = old - 1e-6
            lm = loss()
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / 2e-6
        err = np.max(np.abs(fd - gr[gname])) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_bwd_prologue_identity_taps_and_no_norm_change_nothing():
    # taps (0, 0, 0, 1) make the convolution the identity: every gradient equals the plain one's, and the
    # taps' gradient of the current-token tap is sum_t dL/dy_t x_t
    rng = np.random.default_rng(52)
    B, T, H, K, V = 2, 5, 1, 3, 2
    x, do, dsf = _inputs(rng, B, T, H, K, V)
    w = np.zeros((H, 2 * K + V, 4))
    w[..., 3] = 1.0
    ref = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf)
    gr = oracle.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, conv="short4", conv_w=w)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        assert np.allclose(gr[n], ref[n], rtol=0, atol=1e-12), n
    tap3 = np.concatenate([np.einsum("bthc,bthc->hc", ref["dq"], x["q"]), np.einsum("bthc,bthc->hc", ref["dk"], x["k"]),
                           np.einsum("bthc,bthc->hc", ref["dv"], x["v"])], axis=1)
    assert np.allclose(gr["dconv_w"][..., 3], tap3, rtol=1e-12, atol=1e-12)


PROLOGUE_MISTAKES = ["norm_without_projection", "silu_derivative_dropped", "no_restart_at_sequences",
                     "taps_gradient_transposed"]


@pytest.mark.parametrize("kind", PROLOGUE_MISTAKES)
def test_planted_prologue_mistakes_fail_the_finite_difference_pin(kind, monkeypatch):
    # the prologue's reverse with one planted mistake: some gradient moves off the central differences of the
    # forward oracle by more than 1e-3 (relative), where the correct reverse is within 1e-7
    import oracle.backward as ob
    rng = np.random.default_rng(53)
    B, T, H, K, V = 1, 7, 2, 3, 2
    cu = [0, 3, 7]
    x, do, dsf = _inputs(rng, B, T, H, K, V, 2)
    x["q"] = rng.standard_normal((B, T, H, K))
    x["k"] = rng.standard_normal((B, T, H, K))
    x["w"] = 0.7 * rng.standard_normal((H, 2 * K + V, 4))
    kw = dict(qk_norm=True, conv="short4_silu", conv_w=x["w"])
    good_conv_back = ob._conv_back
    if kind == "norm_without_projection":
        monkeypatch.setattr(ob, "_norm_back", lambda xn, r, dxn: r * dxn)
    elif kind == "silu_derivative_dropped":
        monkeypatch.setattr(ob, "_conv_back", lambda x_, w_, dz, st, act: good_conv_back(x_, w_, dz, st, "short4"))
    elif kind == "no_restart_at_sequences":
        monkeypatch.setattr(ob, "_conv_back",
                            lambda x_, w_, dz, st, act: good_conv_back(x_, w_, dz, np.zeros_like(st), act))
    else:
        def flipped(x_, w_, dz, st, act):
            dx, dw = good_conv_back(x_, w_, dz, st, act)
            return dx, dw[:, :, ::-1].copy()
        monkeypatch.setattr(ob, "_conv_back", flipped)
    gr = ob.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["S0"], dsf, cu, **kw)

    def loss():
        o, sf = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], cu, **kw)
        return float(np.sum(o * do) + np.sum(sf * dsf))
    worst = 0.0
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("w", "dconv_w")):
        fd = np.zeros_like(x[name])
        flat = x[name].reshape(-1)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 1e-6
            lp = loss()
            flat[i] = old - 1e-6
            lm = loss()
            flat[i] = old
            fd.reshape(-1)[i] = (lp - lm) / 2e-6
        worst = max(worst, np.max(np.abs(fd - gr[gname])) / max(1.0, np.max(np.abs(fd))))
    assert worst > 1e-3, (kind, worst)
