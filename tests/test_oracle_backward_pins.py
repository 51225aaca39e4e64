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
