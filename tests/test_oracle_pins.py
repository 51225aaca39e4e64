"""CPU tests: the fp64 oracle against its pins (closed forms, independent
formulations, invariants), plus planted mistakes that the pins must catch."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import kda_pins

HERE = os.path.dirname(os.path.abspath(__file__))


def run_oracle(q, k, v, g, beta, S0, cu):
    return oracle.chunk_fwd(q, k, v, g, beta, S0=S0, cu_seqlens=cu, threads=2)


@pytest.mark.parametrize("pin", kda_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(run_oracle, np.random.default_rng(1234))


def test_exact_bruteforce():
    kda_pins.pin_exact_bruteforce(run_oracle, seeds=(1, 2, 3, 4))


def test_decode_equals_prefill():
    """n decode steps from S equal one prefill of those n tokens started at S."""
    rng = np.random.default_rng(7)
    N, H, K, V, n = 3, 2, 5, 4, 6
    q, k, v, g, beta = kda_pins._rand_problem(rng, N, n, H, K, V)
    S0 = rng.standard_normal((N, H, K, V))
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, g, beta, S0=S0)
    S = S0.copy()
    for t in range(n):
        o_t, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert kda_pins.rel_err(o_t, o_ref[:, t]) < 1e-13
    assert kda_pins.rel_err(S, S_ref) < 1e-13


def test_golden_exact_fixture():
    """Stored exact-rational result of a hand-sized problem (tests/golden)."""
    with open(os.path.join(HERE, "golden", "tiny_exact.json")) as f:
        fx = json.load(f)
    to = lambda m: np.array([[float(Fraction(x)) for x in row] for row in m])
    q, k, v = to(fx["q"]), to(fx["k"]), to(fx["v"])
    alpha = to(fx["alpha"])
    beta = np.array([float(Fraction(x)) for x in fx["beta"]])
    S0 = to(fx["S0"])
    o, Sf = oracle.chunk_fwd(q[None, :, None], k[None, :, None], v[None, :, None], np.log(alpha)[None, :, None],
                             beta[None, :, None], S0=S0[None, None])
    assert kda_pins.rel_err(o[0, :, 0], to(fx["o"])) < 1e-13
    assert kda_pins.rel_err(Sf[0, 0], to(fx["S_final"])) < 1e-13


def test_threads_do_not_change_results():
    rng = np.random.default_rng(11)
    q, k, v, g, beta = kda_pins._rand_problem(rng, 2, 17, 5, 6, 4)
    a = oracle.chunk_fwd(q, k, v, g, beta, threads=1)
    b = oracle.chunk_fwd(q, k, v, g, beta, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_bad_arguments():
    z = np.zeros((1, 4, 1, 2))
    with pytest.raises(ValueError):
        oracle.chunk_fwd(z, z, z, z, np.zeros((1, 4, 1)), cu_seqlens=np.array([0, 3]))  # cu[-1] != T
    with pytest.raises(ValueError):
        oracle.chunk_fwd(z, z, z[..., :1], z, np.zeros((1, 5, 1)))


# ------------------------------------------------------------ the scaled-sigmoid gate

def test_gate_closed_forms():
    """-5 * sigmoid(x) at points where the sigmoid has exact values: 1/2 at 0, 3/4 at ln 3, 1/4 at
    -ln 3, 1/(1+e) at -1; saturation at both ends without NaN."""
    g = oracle.scaled_sigmoid_gate
    assert g(np.array([0.0]))[0] == -2.5
    assert abs(g(np.array([np.log(3.0)]))[0] + 3.75) < 1e-15
    assert abs(g(np.array([-np.log(3.0)]))[0] + 1.25) < 1e-15
    assert abs(g(np.array([-1.0]))[0] + 5.0 / (1.0 + np.e)) < 1e-15
    hi, lo = g(np.array([800.0, 40.0])), g(np.array([-800.0, -40.0]))
    assert hi[0] == -5.0 and abs(hi[1] + 5.0) < 1e-16
    assert lo[0] == 0.0 and -5e-17 < lo[1] < 0.0
    assert not np.isnan(g(np.array([-1e308, 1e308]))).any()


def test_gate_symmetry_range_and_order():
    """sigmoid(x) + sigmoid(-x) = 1, so g(x) + g(-x) = -5; g is strictly decreasing with range (-5, 0)."""
    x = np.sort(np.random.default_rng(5).standard_normal(2001) * 6.0)
    g = oracle.scaled_sigmoid_gate(x)
    assert np.max(np.abs(g + oracle.scaled_sigmoid_gate(-x) + 5.0)) < 1e-14
    assert np.all(np.diff(g) < 0.0)
    assert np.all((g > -5.0) & (g < 0.0))


def test_gate_drives_the_decay():
    """Through the recurrence: with beta = 0 nothing is written, so S_final = diag(prod_t e^(g_t)) S0
    and o_t = (decayed S)^T q_t. At x = 0 every token retains e^(-2.5) of each row; at x = ln 3
    e^(-3.75); a row whose x is very negative keeps S0 unchanged (the gate's upper end)."""
    T, K, V = 5, 3, 2
    rng = np.random.default_rng(17)
    x = np.zeros((1, T, 1, K))
    x[..., 1] = np.log(3.0)
    x[..., 2] = -800.0
    q = rng.standard_normal((1, T, 1, K))
    k = rng.standard_normal((1, T, 1, K))
    v = rng.standard_normal((1, T, 1, V))
    S0 = rng.standard_normal((1, 1, K, V))
    o, Sf = oracle.chunk_fwd(q, k, v, x, np.zeros((1, T, 1)), S0=S0, gate="scaled_sigmoid")
    rate = np.array([-2.5, -3.75, 0.0])
    for t in range(T):
        St = np.exp(rate * (t + 1))[:, None] * S0[0, 0]
        assert kda_pins.rel_err(o[0, t, 0], St.T @ q[0, t, 0]) < 1e-13
    assert kda_pins.rel_err(Sf[0, 0], np.exp(rate * T)[:, None] * S0[0, 0]) < 1e-13
    o_d, S_d = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], x[:, 0], np.zeros((1, 1)), S0, gate="scaled_sigmoid")
    assert kda_pins.rel_err(S_d[0, 0], np.exp(rate)[:, None] * S0[0, 0]) < 1e-13
    with pytest.raises(ValueError):
        oracle.chunk_fwd(q, k, v, x, np.zeros((1, T, 1)), gate="softplus")


# ------------------------------------------------------------ the output gate

def test_output_gate_closed_forms():
    """o * sigmoid(z): z = 0 halves o exactly; sigmoid(z) + sigmoid(-z) = 1, so the outputs under z and -z
    add up to the ungated output; z = ln 3 keeps 3/4; the ends saturate to o and 0; S_final does not depend
    on the gate. Through both the prefill and the decode entry points."""
    rng = np.random.default_rng(23)
    B, T, H, K, V = 1, 9, 2, 4, 3
    q, k, v, g, beta = kda_pins._rand_problem(rng, B, T, H, K, V)
    S0 = rng.standard_normal((B, H, K, V))
    o, Sf = oracle.chunk_fwd(q, k, v, g, beta, S0=S0)
    z = rng.standard_normal((B, T, H, V)) * 3.0
    o0, Sf0 = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=np.zeros_like(z))
    assert np.array_equal(o0, 0.5 * o) and np.array_equal(Sf0, Sf)
    op, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=z)
    om, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=-z)
    assert kda_pins.rel_err(op + om, o) < 1e-14
    o3, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=np.full_like(z, np.log(3.0)))
    assert kda_pins.rel_err(o3, 0.75 * o) < 1e-15
    ohi, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=np.full_like(z, 800.0))
    olo, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, o_gate=np.full_like(z, -800.0))
    assert np.array_equal(ohi, o) and np.all(olo == 0.0)
    od, Sd = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0)
    odz, Sdz = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, o_gate=np.zeros_like(z[:, 0]))
    assert np.array_equal(odz, 0.5 * od) and np.array_equal(Sdz, Sd)
    with pytest.raises(ValueError):
        oracle.chunk_fwd(q, k, v, g, beta, o_gate=z[..., :2])


# ------------------------------------------------------------ the q/k L2 normalisation

def test_l2norm_closed_forms():
    """(3, 4) -> (3/5, 4/5) and (0, -2, 0) -> (0, -1, 0) up to eps; an all-zero vector stays zero (no NaN);
    the direction is kept and the norm of a result is sqrt(n2 / (n2 + eps)) for |x|^2 = n2."""
    f = oracle.l2_normalize
    eps = oracle.L2NORM_EPS
    assert np.allclose(f(np.array([3.0, 4.0])), [0.6, 0.8], rtol=0, atol=1e-7)
    assert np.allclose(f(np.array([0.0, -2.0, 0.0])), [0.0, -1.0, 0.0], rtol=0, atol=1e-6)
    z = f(np.zeros((2, 5)))
    assert np.all(z == 0.0)
    x = np.random.default_rng(41).standard_normal((7, 3, 16)) * 4.0
    y = f(x)
    n2 = np.sum(x * x, axis=-1)
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - np.sqrt(n2 / (n2 + eps)))) < 1e-14
    cos = np.sum(x * y, axis=-1) / (np.linalg.norm(x, axis=-1) * np.linalg.norm(y, axis=-1))
    assert np.max(np.abs(cos - 1.0)) < 1e-14


def test_l2norm_read_after_write_with_raw_keys():
    """With the normalisation on, beta = 1 and q_t = c_t k_t for any unnormalised k_t and any c_t > 0,
    every output equals v_t for any S0 and g (the read-after-write identity, which needs a unit key):
    o_t = S_t^T k^ = (D S)^T k^ - (D S)^T k^ + v_t |k^|^2, and |k^|^2 = 1 up to eps / |k|^2.
    Without the normalisation the same inputs miss it by the factor c_t |k_t|^2."""
    rng = np.random.default_rng(42)
    B, T, H, K, V = 1, 11, 2, 8, 5
    k = rng.standard_normal((B, T, H, K)) * 3.0
    c = np.exp(rng.standard_normal((B, T, H, 1)))
    q = c * k
    v = rng.standard_normal((B, T, H, V))
    g = -5.0 * rng.random((B, T, H, K))
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, K, V))
    o, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, qk_norm=True)
    n2 = np.sum(k * k, axis=-1, keepdims=True)
    assert np.max(np.abs(o - v)) < 1e-6 * np.max(np.abs(v)) + 10 * oracle.L2NORM_EPS / np.min(n2)
    o_raw, _ = oracle.chunk_fwd(q, k, v, g, beta, S0=S0)
    assert np.max(np.abs(o_raw - v)) > 1.0
    od, _ = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, qk_norm=True)
    assert np.max(np.abs(od - v[:, 0])) < 1e-6


def test_l2norm_scale_invariance():
    """Scaling every q and k row by its own positive factor leaves o and S_final unchanged when the
    normalisation is on (to the eps term, ~eps / |k|^2 relative), through prefill and decode; and the
    normalised call equals the plain call on unit-norm rows scaled back (q, k on the sphere)."""
    rng = np.random.default_rng(43)
    B, T, H, K, V = 2, 13, 3, 6, 4
    q, k, v, g, beta = kda_pins._rand_problem(rng, B, T, H, K, V)
    q = q * 10.0
    k = k * 10.0
    S0 = rng.standard_normal((B, H, K, V))
    cq = np.exp(rng.uniform(0.0, 1.5, (B, T, H, 1)))
    ck = np.exp(rng.uniform(0.0, 1.5, (B, T, H, 1)))
    o1, S1 = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, qk_norm=True)
    o2, S2 = oracle.chunk_fwd(cq * q, ck * k, v, g, beta, S0=S0, qk_norm=True)
    assert kda_pins.rel_err(o2, o1) < 1e-6 and kda_pins.rel_err(S2, S1) < 1e-6
    un = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    o3, S3 = oracle.chunk_fwd(un(q), un(k), v, g, beta, S0=S0)
    assert kda_pins.rel_err(o3, o1) < 1e-6 and kda_pins.rel_err(S3, S1) < 1e-6
    od1, Sd1 = oracle.decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, qk_norm=True)
    od2, Sd2 = oracle.decode_step(3.0 * q[:, 0], 0.5 * k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0, qk_norm=True)
    assert kda_pins.rel_err(od2, od1) < 1e-6 and kda_pins.rel_err(Sd2, Sd1) < 1e-6


# ------------------------------------------------------------ the short convolution

def test_short_conv_closed_forms():
    """Taps (0,0,0,1) give x back; taps (0,0,1,0) give the previous token, zero at every sequence start;
    taps (1,1,1,1) give the running sum of the last four tokens of the sequence. Against a direct
    numpy.convolve per channel and sequence (an independent formulation) for random taps."""
    rng = np.random.default_rng(51)
    T, H, D = 23, 2, 5
    x = rng.standard_normal((T, H, D))
    cu = [0, 1, 7, 7, 23]
    st = np.zeros(T, dtype=np.int64)
    for a, b in zip(cu[:-1], cu[1:]):
        st[a:b] = a
    ident = np.zeros((H, D, 4)); ident[..., 3] = 1.0
    assert np.array_equal(oracle.short_conv(x, ident, st), x)
    shift = np.zeros((H, D, 4)); shift[..., 2] = 1.0
    y = oracle.short_conv(x, shift, st)
    for t in range(T):
        assert np.array_equal(y[t], x[t - 1] if t - 1 >= st[t] else np.zeros((H, D)))
    ones = np.ones((H, D, 4))
    y = oracle.short_conv(x, ones, st)
    for t in range(T):
        ref = sum(x[tau] for tau in range(max(st[t], t - 3), t + 1))
        assert np.max(np.abs(y[t] - ref)) < 1e-14
    w = rng.standard_normal((H, D, 4))
    y = oracle.short_conv(x, w, st)
    for a, b in zip(cu[:-1], cu[1:]):
        if a == b:
            continue
        for h in range(H):
            for c in range(D):
                ref = np.convolve(x[a:b, h, c], w[h, c, ::-1])[: b - a]
                assert np.max(np.abs(y[a:b, h, c] - ref), initial=0.0) < 1e-13


def test_silu_closed_forms():
    """silu(0) = 0, silu(ln 3) = (3/4) ln 3, silu(x) - silu(-x) = x, silu -> x and -> 0 at the ends."""
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([np.log(3.0)]))[0] - 0.75 * np.log(3.0)) < 1e-15
    x = np.random.default_rng(52).standard_normal(100) * 4
    assert np.max(np.abs(oracle.silu(x) - oracle.silu(-x) - x)) < 1e-13
    assert oracle.silu(np.array([800.0]))[0] == 800.0 and oracle.silu(np.array([-800.0]))[0] == 0.0


def test_conv_through_prefill_and_decode():
    """Identity taps leave prefill unchanged; with random taps, a prefill with the conv equals a plain
    prefill on inputs convolved by short_conv; and decode steps that carry the 3-token cache reproduce
    the prefill's outputs, state and (from the raw tokens) cache, with and without SiLU, per sequence."""
    rng = np.random.default_rng(53)
    B, T, H, K, V = 1, 13, 2, 4, 3
    q, k, v, g, beta = kda_pins._rand_problem(rng, B, T, H, K, V)
    S0 = rng.standard_normal((2, H, K, V))
    cu = [0, 6, 13]
    ident = np.zeros((H, 2 * K + V, 4)); ident[..., 3] = 1.0
    o0, S_0 = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, cu_seqlens=cu)
    o1, S_1 = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, cu_seqlens=cu, conv="short4", conv_w=ident)
    assert np.array_equal(o0, o1) and np.array_equal(S_0, S_1)
    w = rng.standard_normal((H, 2 * K + V, 4)) * 0.5
    for act in ("short4", "short4_silu"):
        o, Sf = oracle.chunk_fwd(q, k, v, g, beta, S0=S0, cu_seqlens=cu, conv=act, conv_w=w, qk_norm=True)
        st = np.array([0] * 6 + [6] * 7)
        qc = oracle.short_conv(q[0], w[:, :K], st, act)[None]
        kc = oracle.short_conv(k[0], w[:, K:2 * K], st, act)[None]
        vc = oracle.short_conv(v[0], w[:, 2 * K:], st, act)[None]
        o2, S2 = oracle.chunk_fwd(qc, kc, vc, g, beta, S0=S0, cu_seqlens=cu, qk_norm=True)
        assert kda_pins.rel_err(o, o2) < 1e-14 and kda_pins.rel_err(Sf, S2) < 1e-14
        for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
            S = S0[n:n + 1]
            cache = np.zeros((1, H, 3, 2 * K + V))
            for t in range(a, b):
                sl = (slice(0, 1), t)
                od, S, cache = oracle.decode_step(q[sl], k[sl], v[sl], g[sl], beta[sl], S, conv=act, conv_w=w,
                                                  conv_cache=cache, qk_norm=True)
                assert kda_pins.rel_err(od[0], o[0, t]) < 1e-13
            assert kda_pins.rel_err(S, Sf[n:n + 1]) < 1e-13
            raw = np.concatenate([q[0], k[0], v[0]], axis=-1)
            last = [raw[t] if t >= a else np.zeros((H, 2 * K + V)) for t in range(b - 3, b)]
            assert np.array_equal(cache[0], np.stack(last, axis=1))
    with pytest.raises(ValueError):
        oracle.chunk_fwd(q, k, v, g, beta, conv="short4", conv_w=w[:, :K])


# ------------------------------------------------------------ planted mistakes
#
# A small numpy re-implementation with switches for plausible mistakes. The
# correct switch setting must pass every pin; each mistake must fail at least
# one pin. This shows the pins constrain the oracle's arithmetic.

def make_runner(mistake=None):
    def run(q, k, v, g, beta, S0, cu):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        B, T, H, K = q.shape
        V = v.shape[-1]
        if cu is None:
            seqs = [(n, n * T, (n + 1) * T) for n in range(B)]
        else:
            seqs = [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
        qf, kf, gf = (x.reshape(B * T, H, K) for x in (q, k, g))
        vf = v.reshape(B * T, H, V)
        bf = beta.reshape(B * T, H)
        o = np.zeros((B * T, H, V))
        Sf = np.zeros((len(seqs), H, K, V))
        carry = None
        for n, t0, t1 in seqs:
            for h in range(H):
                S = np.zeros((K, V)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
                if mistake == "no_reset" and carry is not None and h == 0:
                    S = carry.copy()
                for t in range(t0, t1):
                    kt, vt, qt, bt = kf[t, h], vf[t, h], qf[t, h], bf[t, h]
                    gt = gf[t - 1, h] if (mistake == "gate_index" and t > t0) else gf[t, h]
                    a = gt if mistake == "alpha_is_g" else np.exp(gt)
                    if mistake == "read_before_decay":
                        u = S.T @ kt
                        S = a[:, None] * S
                    elif mistake == "decay_after_write":
                        u = S.T @ kt
                    else:
                        S = (a[:V][None, :] * S) if mistake == "decay_columns" else a[:, None] * S
                        u = S.T @ (qt if mistake == "query_reads" else kt)
                    if mistake == "transposed_read":
                        u = S @ kt[:V]
                    if mistake == "sign_flip":
                        S_new = S + bt * np.outer(kt, vt + u)
                    elif mistake == "beta_on_value_only":
                        S_new = S + np.outer(kt, bt * vt - u)
                    elif mistake == "beta_squared":
                        S_new = S + bt * bt * np.outer(kt, vt - u)
                    else:
                        S_new = S + bt * np.outer(kt, vt - u)
                    if mistake == "decay_after_write":
                        S_new = a[:, None] * S_new
                    o[t, h] = (S if mistake == "read_old_state" else S_new).T @ qt
                    S = S_new
                Sf[n, h] = S
                if h == 0:
                    carry = S
        return o.reshape(B, T, H, V), Sf
    return run


MISTAKES = ["read_before_decay", "decay_after_write", "read_old_state", "sign_flip", "beta_on_value_only",
            "beta_squared", "decay_columns", "alpha_is_g", "query_reads", "transposed_read", "gate_index",
            "no_reset"]


def _fails_some_pin(run):
    for pin in kda_pins.ALL_PINS:
        try:
            pin(run, np.random.default_rng(99))
        except Exception:
            return pin.__name__
    try:
        kda_pins.pin_exact_bruteforce(run, seeds=(1,))
    except Exception:
        return "pin_exact_bruteforce"
    return None


def test_correct_reimplementation_passes_pins():
    assert _fails_some_pin(make_runner(None)) is None


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    assert _fails_some_pin(make_runner(mistake)) is not None, mistake
