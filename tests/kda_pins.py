"""Pins for the KDA oracle: closed forms, special cases, invariants and
independent formulations that a plausible mistake in the recurrence breaks.

Each pin takes ``run(q, k, v, g, beta, S0, cu_seqlens) -> (o, S_final)`` with
numpy float64 arrays in the layouts [B,T,H,K] / [B,T,H,V] / [B,T,H] /
[N,H,K,V], so the same pins check the C oracle and, in the planted-mistake
test, deliberately broken variants.

Sources of the facts pinned (page titles as published):
  [P4] "Kimi K3 发布核实与 Moonshot AI 主干架构演变", section 3, paragraph
       "KDA 为什么不同于 MLA": decay by per-channel retention first, then the
       beta/key/value correction; the query reads the updated state; training
       may run recurrent across chunks and parallel inside a chunk.
  [P2] "Kimi K3 模型架构解析：KDA、AttnRes 与 Stable LatentMoE", section 二.3
       "Delta Rule：写入新记忆前修正旧映射": read the stored mapping with the key,
       form the error against the value, write back only the difference.
"""
from __future__ import annotations

import numpy as np

from oracle.exact import rational_problem, transition_form

TOL = 1e-12  # fp64 arithmetic, tiny problems


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(ref)))) if ref.size else 1.0
    return float(np.max(np.abs(x - ref))) / scale if ref.size else 0.0


def _rand_problem(rng, B, T, H, K, V, normalize_k=True, beta=None, g_scale=1.0):
    q = rng.standard_normal((B, T, H, K))
    k = rng.standard_normal((B, T, H, K))
    if normalize_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, K)))) * g_scale
    b = rng.uniform(0.05, 1.0, size=(B, T, H)) if beta is None else np.full((B, T, H), float(beta))
    return q, k, v, g, b


# ---------------------------------------------------------------- closed forms

def pin_passthrough(run, rng):
    """beta = 0 and g = 0: the state is carried unchanged, o_t = S0^T q_t."""
    B, T, H, K, V = 2, 7, 3, 5, 4
    q, k, v, _, _ = _rand_problem(rng, B, T, H, K, V)
    g = np.zeros((B, T, H, K))
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, K, V))
    o, Sf = run(q, k, v, g, beta, S0, None)
    assert np.array_equal(Sf, S0), "passthrough must return S0 exactly"
    o_ref = np.einsum("bthk,bhkv->bthv", q, S0)
    assert rel_err(o, o_ref) < TOL


def pin_pure_decay(run, rng):
    """beta = 0: S_t = diag(exp(sum_{j<=t} g_j)) S0 (rows = key channels)."""
    B, T, H, K, V = 1, 9, 2, 6, 3  # K != V so a decay on the wrong axis cannot even broadcast
    q, k, v, g, _ = _rand_problem(rng, B, T, H, K, V)
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, K, V))
    o, Sf = run(q, k, v, g, beta, S0, None)
    cum = np.cumsum(g, axis=1)  # [B,T,H,K]
    S_t = np.exp(cum)[..., None] * S0[:, None]  # [B,T,H,K,V]
    o_ref = np.einsum("bthk,bthkv->bthv", q, S_t)
    assert rel_err(Sf, S_t[:, -1]) < TOL
    assert rel_err(o, o_ref) < TOL


def pin_single_token(run, rng):
    """One token from S0 = 0: S = beta k v^T and o = beta (k.q) v."""
    B, T, H, K, V = 1, 1, 4, 5, 3
    q, k, v, g, beta = _rand_problem(rng, B, T, H, K, V, normalize_k=False)
    o, Sf = run(q, k, v, g, beta, None, None)
    S_ref = beta[0, 0][:, None, None] * np.einsum("hk,hv->hkv", k[0, 0], v[0, 0])
    o_ref = (beta[0, 0] * np.sum(k[0, 0] * q[0, 0], axis=-1))[:, None] * v[0, 0]
    assert rel_err(Sf[0], S_ref) < TOL
    assert rel_err(o[0, 0], o_ref) < TOL


def pin_read_after_write(run, rng):
    """beta = 1, |k| = 1, q = k gives o_t = v_t for ANY S0 and g.

    With the decayed state D S read by k, the corrected state returns exactly
    v for the same unit key; a read before the decay, a decay after the
    correction, or a read of the old state all break this.
    """
    B, T, H, K, V = 1, 11, 2, 6, 5
    _, k, v, g, _ = _rand_problem(rng, B, T, H, K, V)
    q = k.copy()
    beta = np.ones((B, T, H))
    S0 = rng.standard_normal((B, H, K, V))
    o, _ = run(q, k, v, g, beta, S0, None)
    assert rel_err(o, v) < 1e-11


def pin_exact_recall(run, rng):
    """beta = 1, g = 0, S0 = 0 and orthonormal keys: S_T = K^T V and q = k_j recalls v_j."""
    K, V, T, H = 8, 6, 8, 2
    keys = np.stack([np.linalg.qr(rng.standard_normal((K, K)))[0].T[:T] for _ in range(H)], axis=1)  # [T,H,K]
    v = rng.standard_normal((1, T, H, V))
    k = keys[None]
    g = np.zeros((1, T, H, K))
    beta = np.ones((1, T, H))
    q = np.zeros((1, T, H, K))
    _, Sf = run(q, k, v, g, beta, None, None)
    S_ref = np.einsum("thk,thv->hkv", keys, v[0])
    assert rel_err(Sf[0], S_ref) < TOL
    recalled = np.einsum("thk,hkv->thv", keys, Sf[0])
    assert rel_err(recalled, v[0]) < TOL


# ------------------------------------------------ independent formulations

def chunked_wy(q, k, v, g, beta, S0, C):
    """Chunk-parallel form for ONE (sequence, head), written from the algebra.

    Inside a chunk with cumulative log-decay b_r (per key channel) and
    Gamma_r = exp(b_r):
      A = tril_strict(diag(beta) (K*Gamma)(K/Gamma)^T)
      T = (I + A)^{-1} diag(beta)          (numpy.linalg.solve)
      W = T V - T (K*Gamma) S              (the corrected writes)
      O = (Q*Gamma) S + tril((Q*Gamma)(K/Gamma)^T) W
      S <- diag(Gamma_C) S + (K * Gamma_C/Gamma)^T W
    Shapes: q, k, g [T,K]; v [T,V]; beta [T]; S0 [K,V].
    """
    Tn, K = k.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((Tn, v.shape[1]))
    for c0 in range(0, Tn, C):
        sl = slice(c0, min(Tn, c0 + C))
        kc, qc, vc, gc, bc = k[sl], q[sl], v[sl], g[sl], beta[sl]
        L = kc.shape[0]
        b = np.cumsum(gc, axis=0)
        Gam = np.exp(b)
        A = np.tril(bc[:, None] * ((kc * Gam) @ (kc / Gam).T), -1)
        Tm = np.linalg.solve(np.eye(L) + A, np.diag(bc))
        W = Tm @ vc - Tm @ (kc * Gam) @ S
        P = np.tril((qc * Gam) @ (kc / Gam).T)
        o[sl] = (qc * Gam) @ S + P @ W
        S = np.exp(b[-1])[:, None] * S + (kc * np.exp(b[-1] - b)).T @ W
    return o, S


def pin_chunked_equivalence(run, rng, chunks=(1, 2, 3, 16, 64)):
    """The chunk-parallel form equals the recurrence for every chunk size."""
    B, T, H, K, V = 2, 70, 2, 7, 5
    q, k, v, g, beta = _rand_problem(rng, B, T, H, K, V)
    S0 = rng.standard_normal((B, H, K, V))
    o, Sf = run(q, k, v, g, beta, S0, None)
    for C in chunks:
        for bb in range(B):
            for h in range(H):
                oc, Sc = chunked_wy(q[bb, :, h], k[bb, :, h], v[bb, :, h], g[bb, :, h], beta[bb, :, h],
                                    S0[bb, h], C)
                assert rel_err(o[bb, :, h], oc) < 1e-10, C
                assert rel_err(Sf[bb, h], Sc) < 1e-10, C


def pin_exact_bruteforce(run, seeds=(1, 2, 3)):
    """Exact rational transition form vs the fp64 oracle on tiny cases."""
    for seed in seeds:
        T, K, V = 6, 3, 2
        q, k, v, alpha, beta, S0 = rational_problem(seed, T, K, V)
        o_ex, S_ex = transition_form(q, k, v, alpha, beta, S0)
        f = lambda m: np.array([[float(x) for x in row] for row in m])
        qa, ka, va = f(q)[None, :, None], f(k)[None, :, None], f(v)[None, :, None]
        ga = np.log(f(alpha))[None, :, None]
        ba = np.array([float(x) for x in beta])[None, :, None]
        o, Sf = run(qa, ka, va, ga, ba, f(S0)[None, None], None)
        assert rel_err(o[0, :, 0], f(o_ex)) < 1e-12
        assert rel_err(Sf[0, 0], f(S_ex)) < 1e-12


# ---------------------------------------------------------------- invariants

def pin_linearity(run, rng):
    """(o, S_final) is jointly linear in (V, S0) for fixed q, k, g, beta."""
    B, T, H, K, V = 1, 13, 2, 4, 3
    q, k, v1, g, beta = _rand_problem(rng, B, T, H, K, V)
    v2 = rng.standard_normal(v1.shape)
    S1 = rng.standard_normal((B, H, K, V))
    S2 = rng.standard_normal((B, H, K, V))
    a, b = 0.7, -1.3
    o1, F1 = run(q, k, v1, g, beta, S1, None)
    o2, F2 = run(q, k, v2, g, beta, S2, None)
    o3, F3 = run(q, k, a * v1 + b * v2, g, beta, a * S1 + b * S2, None)
    assert rel_err(o3, a * o1 + b * o2) < TOL
    assert rel_err(F3, a * F1 + b * F2) < TOL


def pin_split_resume(run, rng):
    """Two calls chained through S_final equal one call over the whole sequence."""
    B, T, H, K, V = 2, 20, 2, 5, 4
    q, k, v, g, beta = _rand_problem(rng, B, T, H, K, V)
    S0 = rng.standard_normal((B, H, K, V))
    o, Sf = run(q, k, v, g, beta, S0, None)
    s = 7
    oa, Sa = run(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], S0, None)
    ob, Sb = run(q[:, s:], k[:, s:], v[:, s:], g[:, s:], beta[:, s:], Sa, None)
    assert rel_err(np.concatenate([oa, ob], axis=1), o) < TOL
    assert rel_err(Sb, Sf) < TOL


def pin_varlen(run, rng):
    """A packed batch with cu_seqlens equals separate per-sequence calls, and
    the state restarts from S0[n] at every sequence boundary (also for empty sequences)."""
    lengths = [5, 0, 9, 1, 4]
    H, K, V = 2, 4, 3
    T = sum(lengths)
    q, k, v, g, beta = _rand_problem(rng, 1, T, H, K, V)
    S0 = rng.standard_normal((len(lengths), H, K, V))
    cu = np.cumsum([0] + lengths).astype(np.int64)
    o, Sf = run(q, k, v, g, beta, S0, cu)
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        on, Sn = run(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], S0[n:n + 1], None)
        assert rel_err(o[:, a:b], on) < TOL
        assert rel_err(Sf[n:n + 1], Sn) < TOL
    assert np.array_equal(Sf[1], S0[1]), "an empty sequence returns its S0"


def pin_head_permutation(run, rng):
    """Permuting heads permutes outputs (heads are independent)."""
    B, T, H, K, V = 1, 9, 4, 3, 3
    q, k, v, g, beta = _rand_problem(rng, B, T, H, K, V)
    S0 = rng.standard_normal((B, H, K, V))
    perm = np.array([2, 0, 3, 1])
    o, Sf = run(q, k, v, g, beta, S0, None)
    op, Sp = run(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm], beta[:, :, perm], S0[:, perm], None)
    assert rel_err(op, o[:, :, perm]) < TOL
    assert rel_err(Sp, Sf[:, perm]) < TOL


def pin_contraction_bound(run, rng):
    """With |k| = 1, 0 <= beta <= 1 and g <= 0 the spectral norm grows by at most
    beta_t |v_t| per token (I - beta k k^T and the decay are contractions)."""
    B, T, H, K, V = 1, 1, 1, 6, 5
    S = rng.standard_normal((B, H, K, V))
    for t in range(25):
        q, k, v, g, beta = _rand_problem(rng, B, T, H, K, V)
        _, Sn = run(q, k, v, g, beta, S, None)
        lhs = np.linalg.norm(Sn[0, 0], 2)
        rhs = np.linalg.norm(S[0, 0], 2) + beta[0, 0, 0] * np.linalg.norm(v[0, 0, 0])
        assert lhs <= rhs * (1 + 1e-12)
        S = Sn


ALL_PINS = [pin_passthrough, pin_pure_decay, pin_single_token, pin_read_after_write, pin_exact_recall,
            pin_chunked_equivalence, pin_linearity, pin_split_resume, pin_varlen, pin_head_permutation,
            pin_contraction_bound]


def run_all(run, seed=0):
    for pin in ALL_PINS:
        pin(run, np.random.default_rng(seed))
    pin_exact_bruteforce(run)
