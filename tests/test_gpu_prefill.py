"""GPU parity of kda_chunk_fwd (through the C ABI) against the fp64 oracle.

Every case prints its name, seed and shape before touching the GPU. Inputs
come from the seeded generator; the oracle sees exactly the values the GPU
received (bf16 or fp32), widened to fp64.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_gated_delta_chunk_amd import chunk_fwd
from kda_gated_delta_chunk_amd import synth
from tests.parity import TOL_BF16, TOL_FP32, err, err_stored

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(name, **kw):
    print("\n[case] %s %s" % (name, " ".join("%s=%s" % kv for kv in kw.items())), flush=True)


def _oracle(inp, heads=None):
    q, k, v, g, beta, S0, cu = (inp[n] for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens"))
    if heads is not None:
        hs = list(heads)
        q, k, v, g, beta = (x[:, :, hs].contiguous() for x in (q, k, v, g, beta))
        S0 = None if S0 is None else S0[:, hs].contiguous()
    return oracle.chunk_fwd(q.cpu(), k.cpu(), v.cpu(), g.cpu(), beta.cpu(), None if S0 is None else S0.cpu(),
                            None if cu is None else cu.cpu())


def _run(inp, o_dtype=None):
    o, Sf = chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S0=inp["S0"],
                      cu_seqlens=inp["cu_seqlens"], o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, Sf


def _check(inp, heads=None, io="bf16", written=None):
    """Run the GPU path (and for bf16 also with fp32 o) and compare with the oracle."""
    o_ref, S_ref = _oracle(inp, heads)
    o, Sf = _run(inp)
    sel = (lambda x: x[:, :, list(heads)]) if heads is not None else (lambda x: x)
    selS = (lambda x: x[:, list(heads)]) if heads is not None else (lambda x: x)
    o_c = sel(o).cpu()
    if written is not None:  # only tokens inside a sequence are written
        o_c, o_ref = o_c[:, written], o_ref[:, written]
    res = {"S": err(selS(Sf).cpu(), S_ref)}
    if io == "fp32":
        res["o"] = err(o_c, o_ref)
        print("  errors", res, flush=True)
        assert res["o"] <= TOL_FP32 and res["S"] <= TOL_FP32, res
        return o, Sf
    o32, Sf32 = _run(inp, o_dtype=torch.float32)
    o32_c = sel(o32).cpu()
    if written is not None:
        o32_c = o32_c[:, written]
    res["o_fp32"] = err(o32_c, o_ref)
    res["o_bf16_stored"] = err_stored(o_c, o_ref)
    print("  errors", res, flush=True)
    # the bf16 store is exactly the round-to-nearest-even of the fp32 result
    assert torch.equal(o32_c.to(torch.bfloat16), o_c)
    assert torch.equal(Sf32, Sf)
    assert res["o_fp32"] <= TOL_BF16 and res["S"] <= TOL_BF16 and res["o_bf16_stored"] <= TOL_BF16, res
    return o, Sf


@pytest.fixture(scope="module", autouse=True)
def _threads():
    torch.manual_seed(0)
    yield


def test_tiny_fp32_workload():
    """B=1, H=2, T=64, K=V=32, chunk 16, fp32 I/O, zero initial state."""
    w = synth.WORKLOADS["tiny_fp32"]
    _announce("tiny_fp32", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp, io="fp32")


@pytest.mark.parametrize("B,T,H,K,V", [(2, 77, 3, 128, 128), (1, 50, 2, 64, 32), (1, 33, 2, 32, 128),
                                       (1, 16, 1, 128, 64), (3, 5, 2, 32, 32)])
def test_fp32_shapes_with_state(B, T, H, K, V):
    _announce("fp32_shapes", B=B, T=T, H=H, K=K, V=V, seed=11)
    inp = synth.prefill_inputs(B, T, H, K, V, "fp32", seed=11, device=DEV, with_S0=True)
    _check(inp, io="fp32")


@pytest.mark.parametrize("B,T,H,K,V", [(2, 200, 3, 128, 128), (1, 97, 2, 64, 64), (1, 48, 4, 32, 128),
                                       (2, 31, 2, 128, 32)])
def test_bf16_shapes_with_state(B, T, H, K, V):
    _announce("bf16_shapes", B=B, T=T, H=H, K=K, V=V, seed=12)
    inp = synth.prefill_inputs(B, T, H, K, V, "bf16", seed=12, device=DEV, with_S0=True)
    _check(inp)


def test_bf16_varlen_with_empty_and_ragged_sequences():
    lengths = [37, 0, 16, 1, 150, 64, 0]
    cu = synth.cu_from_lengths(lengths)
    _announce("bf16_varlen", lengths=lengths, seed=13)
    inp = synth.prefill_inputs(1, cu[-1], 4, 64, 64, "bf16", seed=13, device=DEV, cu_seqlens=cu, with_S0=True)
    o, Sf = _check(inp)
    S0 = inp["S0"]
    assert torch.equal(Sf[1], S0[1]) and torch.equal(Sf[6], S0[6]), "empty sequences return S0 exactly"


def test_fp32_varlen():
    lengths = [5, 0, 17, 32, 3]
    cu = synth.cu_from_lengths(lengths)
    _announce("fp32_varlen", lengths=lengths, seed=14)
    inp = synth.prefill_inputs(1, cu[-1], 3, 32, 64, "fp32", seed=14, device=DEV, cu_seqlens=cu, with_S0=True)
    _check(inp, io="fp32")


def test_bf16_mild_decay_long_carry():
    """g = -5 sigmoid(x - 6): alpha ~ 0.988, state carried across many chunks."""
    _announce("bf16_mild_decay", T=1024, H=2, seed=15)
    inp = synth.prefill_inputs(1, 1024, 2, 128, 128, "bf16", seed=15, device=DEV, with_S0=True, g_shift=-6.0)
    _check(inp)


def test_range_edge_and_dense_recall():
    """g = -5 exactly on every channel (e^-80 factors inside a chunk), beta = 1."""
    _announce("range_edge", T=64, H=2, seed=16)
    inp = synth.prefill_inputs(1, 64, 2, 128, 128, "bf16", seed=16, device=DEV, with_S0=True, g_const=-5.0,
                               beta_const=1.0)
    _check(inp)


@pytest.mark.parametrize("io,K,V", [("fp32", 64, 64), ("bf16", 32, 128), ("bf16", 64, 32), ("bf16", 128, 128),
                                     ("fp32", 32, 32)])
def test_passthrough_is_exact(io, K, V):
    """beta = 0, g = 0: S_final is S0 bit for bit and o_t = S0^T q_t in every chunk
    (the state carried into chunks after the first is checked row by row)."""
    _announce("passthrough", io=io, K=K, V=V, T=72, H=2, seed=17)
    inp = synth.prefill_inputs(1, 72, 2, K, V, io, seed=17, device=DEV, with_S0=True, g_const=0.0, beta_const=0.0)
    o, Sf = _run(inp, o_dtype=torch.float32)
    assert torch.equal(Sf, inp["S0"])
    o_ref = torch.einsum("bthk,bhkv->bthv", inp["q"].double().cpu(), inp["S0"].double().cpu())
    assert err(o.cpu(), o_ref) <= (TOL_FP32 if io == "fp32" else TOL_BF16)


def test_zero_and_one_token():
    for T in (0, 1):
        _announce("short", T=T, seed=18)
        inp = synth.prefill_inputs(1, T, 2, 32, 32, "fp32", seed=18, device=DEV, with_S0=True)
        o, Sf = _run(inp)
        if T == 0:
            assert torch.equal(Sf, inp["S0"])
        else:
            _check(inp, io="fp32")


def test_split_resume_matches_one_call():
    _announce("split_resume", T=300, seed=19)
    inp = synth.prefill_inputs(1, 300, 2, 128, 128, "fp32", seed=19, device=DEV, with_S0=True)
    o, Sf = _run(inp)
    s = 123
    a = {n: (x[:, :s].contiguous() if n in ("q", "k", "v", "g", "beta") else x) for n, x in inp.items()}
    oa, Sa = _run(a)
    b = {n: (x[:, s:].contiguous() if n in ("q", "k", "v", "g", "beta") else x) for n, x in inp.items()}
    b["S0"] = Sa
    ob, Sb = _run(b)
    assert err(torch.cat([oa, ob], 1).cpu(), o.cpu()) <= TOL_FP32
    assert err(Sb.cpu(), Sf.cpu()) <= TOL_FP32


@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("K", [32, 64, 128])
@pytest.mark.parametrize("V", [32, 64, 128])
def test_deterministic(io, K, V):
    """Bitwise run-to-run reproducibility (no atomics, no order-dependent reductions),
    over every kernel variant; four repeats so an intermittent race shows up."""
    _announce("deterministic", io=io, K=K, V=V, seed=20)
    inp = synth.prefill_inputs(1, 500, 4, K, V, io, seed=20, device=DEV, with_S0=True)
    o1, S1 = _run(inp, o_dtype=torch.float32)
    for _ in range(3):
        o2, S2 = _run(inp, o_dtype=torch.float32)
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_k3_prefill_4k_all_heads():
    """H=96, T=4096, K=V=128, bf16, chunk 16 (the benchmarked workload), every head."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp)


def test_k3_varlen_16_sampled_heads():
    """16 packed sequences (lengths 256..16384, ~130K tokens), H=96, per-sequence S0;
    the oracle runs on 3 heads, compared with the same heads of the full GPU call."""
    w = synth.WORKLOADS["varlen_16"]
    _announce("varlen_16", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp, heads=(0, 41, 95))
