"""GPU parity of kda_chunk_fwd (through the C ABI) against the fp64 oracle.

Every case prints its name, seed and shape before touching the GPU. Inputs
come from the seeded generator; the oracle sees exactly the values the GPU
received (bf16 or fp32), widened to fp64.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_gated_delta_chunk_amd import (_lib, chunk_fwd, chunk_prep, chunk_state, min_workspace_bytes,
                                       prep_workspace_bytes, synth, workspace_bytes, workspace_status)
from tests.parity import TOL_BF16, TOL_FP32, err, err_stored

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(name, **kw):
    print("\n[case] %s %s" % (name, " ".join("%s=%s" % kv for kv in kw.items())), flush=True)


def _oracle(inp, heads=None):
    q, k, v, g, beta, S0, cu = (inp[n] for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens"))
    og = inp.get("o_gate")
    if heads is not None:
        hs = list(heads)
        q, k, v, g, beta = (x[:, :, hs].contiguous() for x in (q, k, v, g, beta))
        og = None if og is None else og[:, :, hs].contiguous()
        S0 = None if S0 is None else S0[:, hs].contiguous()
    return oracle.chunk_fwd(q.cpu(), k.cpu(), v.cpu(), g.cpu(), beta.cpu(), None if S0 is None else S0.cpu(),
                            None if cu is None else cu.cpu(), gate=inp.get("gate", "log_decay"),
                            o_gate=None if og is None else og.cpu(), qk_norm=inp.get("qk_norm", False),
                            conv=inp.get("conv", "none"), conv_w=_conv_w_heads(inp, heads))


def _conv_w_heads(inp, heads):
    w = inp.get("conv_w")
    if w is None:
        return None
    w = w.cpu()
    return w[list(heads)].contiguous() if heads is not None else w


def _poisoned(shape, dtype):
    """An output buffer filled with NaN: an element the kernels fail to write stays NaN and fails every
    comparison."""
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _run(inp, o_dtype=None, chunk=16, operands=None):
    """One kda_chunk_fwd call with its workspace filled with 0xff bytes (NaN in every float format) and
    o and S_final filled with NaN beforehand, so that no uninitialised byte can pass; the workspace's
    device-side error word must read 0 afterwards."""
    q, v = inp["q"], inp["v"]
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    ops = operands or inp.get("operands", "bf16")
    conv = inp.get("conv", "none")
    need = workspace_bytes(B, T, H, K, V, N, chunk, q.dtype, conv=conv, operands=ops)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    odt = q.dtype if o_dtype is None else o_dtype
    o = _poisoned((B, T, H, V), odt)
    Sf = _poisoned((N, H, K, V), torch.float32)
    chunk_fwd(q, inp["k"], v, inp["g"], inp["beta"], S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], o_dtype=o_dtype,
              chunk=chunk, gate=inp.get("gate", "log_decay"), o_gate=inp.get("o_gate"),
              qk_norm=inp.get("qk_norm", False), conv=conv, conv_w=inp.get("conv_w"), operands=ops,
              workspace=ws, out=o, final_state_out=Sf)
    torch.cuda.synchronize()
    assert workspace_status(ws) == 0, "device-side error recorded in the workspace"
    return o, Sf


def _run_low_memory(inp, o_dtype=None, operands="bf16"):
    """kda_chunk_fwd with only the least workspace it accepts: the fused kernel (16-token chunks, no
    convolution), on poisoned outputs and workspace."""
    q, v = inp["q"], inp["v"]
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    need = min_workspace_bytes(B, T, H, K, V, N, 16, q.dtype, operands=operands)
    assert 0 < need < workspace_bytes(B, T, H, K, V, N, 16, q.dtype, operands=operands)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    odt = q.dtype if o_dtype is None else o_dtype
    o = _poisoned((B, T, H, V), odt)
    Sf = _poisoned((N, H, K, V), torch.float32)
    chunk_fwd(q, inp["k"], v, inp["g"], inp["beta"], S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], o_dtype=o_dtype,
              gate=inp.get("gate", "log_decay"), o_gate=inp.get("o_gate"), qk_norm=inp.get("qk_norm", False),
              operands=operands, workspace=ws, out=o, final_state_out=Sf)
    torch.cuda.synchronize()
    assert workspace_status(ws) == 0, "device-side error recorded in the workspace"
    return o, Sf


def _run_split(inp, chunk=16, operands="bf16", o_dtype=None):
    """kda_chunk_prep then kda_chunk_state on one poisoned workspace (the format travels in its header)."""
    q, v = inp["q"], inp["v"]
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    conv = inp.get("conv", "none")
    need = prep_workspace_bytes(B, T, H, K, V, N, chunk, q.dtype, conv=conv, operands=operands)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    odt = q.dtype if o_dtype is None else o_dtype
    o = _poisoned((B, T, H, V), odt)
    Sf = _poisoned((N, H, K, V), torch.float32)
    chunk_prep(q, inp["k"], inp["g"], inp["beta"], ws, cu_seqlens=inp["cu_seqlens"], V=V, chunk=chunk,
               gate=inp.get("gate", "log_decay"), qk_norm=inp.get("qk_norm", False), conv=conv,
               conv_w=inp.get("conv_w"), operands=operands)
    chunk_state(v, ws, K, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], chunk=chunk, o_dtype=o_dtype, out=o,
                o_gate=inp.get("o_gate"), conv=conv, conv_w=inp.get("conv_w"), final_state_out=Sf)
    torch.cuda.synchronize()
    assert workspace_status(ws) == 0, "device-side error recorded in the workspace"
    return o, Sf, ws


def _check(inp, heads=None, io="bf16", written=None, chunk=16, operands=None):
    """Run the GPU path (and for bf16 also with fp32 o) and compare with the oracle."""
    o_ref, S_ref = _oracle(inp, heads)
    o, Sf = _run(inp, chunk=chunk, operands=operands)
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
    o32, Sf32 = _run(inp, o_dtype=torch.float32, chunk=chunk, operands=operands)
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


CHUNKS = pytest.mark.parametrize("chunk", [16, 64])


@CHUNKS
@pytest.mark.parametrize("B,T,H,K,V", [(2, 77, 3, 128, 128), (1, 50, 2, 64, 32), (1, 33, 2, 32, 128),
                                       (1, 16, 1, 128, 64), (3, 5, 2, 32, 32), (1, 130, 2, 64, 128)])
def test_fp32_shapes_with_state(B, T, H, K, V, chunk):
    _announce("fp32_shapes", B=B, T=T, H=H, K=K, V=V, chunk=chunk, seed=11)
    inp = synth.prefill_inputs(B, T, H, K, V, "fp32", seed=11, device=DEV, with_S0=True)
    _check(inp, io="fp32", chunk=chunk)


@CHUNKS
@pytest.mark.parametrize("gate", ["log_decay", "scaled_sigmoid"])
@pytest.mark.parametrize("T", [77, 128])
def test_fp32_state_at_the_recurrences_precision(chunk, gate, T):
    """fp32 I/O under strong decay (g = -5*sigmoid(N(0,1)), about -2.5 per token and channel): S_final is held
    to 1e-5, ten times tighter than the fp32 bound. A plain fp32 per-token recurrence reaches about 1.4e-6 on
    these inputs. The chunk kernels form the exponent of K*exp(b_C - b) as the sum of the decays after each
    token; formed as the chunk total minus the prefix, it cancels against the total and left 2.4e-5 to 4.9e-5
    at T=77 (1.0e-4 on a 64-token chunk with the sigmoid gate and a convolution). T=128 ends on a whole
    64-token chunk, whose last tokens sit three sub-tiles after its start."""
    _announce("fp32_state_precision", B=2, T=T, H=3, K=128, V=128, chunk=chunk, gate=gate, seed=50)
    if gate == "log_decay":
        inp = synth.prefill_inputs(2, T, 3, 128, 128, "fp32", seed=50, device=DEV, with_S0=True)
    else:
        inp = _gate_inputs(2, T, 3, 128, 128, "fp32", 50, with_S0=True)
    o_ref, S_ref = _oracle(inp)
    o, Sf = _run(inp, chunk=chunk)
    res = {"S": err(Sf.cpu(), S_ref), "o": err(o.cpu(), o_ref)}
    print("  errors", res, flush=True)
    assert res["S"] <= 1e-5 and res["o"] <= TOL_FP32, res


@CHUNKS
@pytest.mark.parametrize("B,T,H,K,V", [(2, 200, 3, 128, 128), (1, 97, 2, 64, 64), (1, 48, 4, 32, 128),
                                       (2, 31, 2, 128, 32), (1, 129, 2, 128, 64)])
def test_bf16_shapes_with_state(B, T, H, K, V, chunk):
    _announce("bf16_shapes", B=B, T=T, H=H, K=K, V=V, chunk=chunk, seed=12)
    inp = synth.prefill_inputs(B, T, H, K, V, "bf16", seed=12, device=DEV, with_S0=True)
    _check(inp, chunk=chunk)


@CHUNKS
def test_bf16_varlen_with_empty_and_ragged_sequences(chunk):
    lengths = [37, 0, 16, 1, 150, 64, 0, 65]
    cu = synth.cu_from_lengths(lengths)
    _announce("bf16_varlen", lengths=lengths, chunk=chunk, seed=13)
    inp = synth.prefill_inputs(1, cu[-1], 4, 64, 64, "bf16", seed=13, device=DEV, cu_seqlens=cu, with_S0=True)
    o, Sf = _check(inp, chunk=chunk)
    S0 = inp["S0"]
    assert torch.equal(Sf[1], S0[1]) and torch.equal(Sf[6], S0[6]), "empty sequences return S0 exactly"


@CHUNKS
def test_fp32_varlen(chunk):
    lengths = [5, 0, 17, 32, 3, 70]
    cu = synth.cu_from_lengths(lengths)
    _announce("fp32_varlen", lengths=lengths, chunk=chunk, seed=14)
    inp = synth.prefill_inputs(1, cu[-1], 3, 32, 64, "fp32", seed=14, device=DEV, cu_seqlens=cu, with_S0=True)
    _check(inp, io="fp32", chunk=chunk)


@CHUNKS
def test_bf16_mild_decay_long_carry(chunk):
    """g = -5 sigmoid(x - 6): alpha ~ 0.988, state carried across many chunks."""
    _announce("bf16_mild_decay", T=1024, H=2, chunk=chunk, seed=15)
    inp = synth.prefill_inputs(1, 1024, 2, 128, 128, "bf16", seed=15, device=DEV, with_S0=True, g_shift=-6.0)
    _check(inp, chunk=chunk)


@CHUNKS
def test_range_edge_and_dense_recall(chunk):
    """g = -5 exactly on every channel (e^-80 factors inside a 16-token tile, e^-320 across a
    64-token chunk), beta = 1."""
    _announce("range_edge", T=160, H=2, chunk=chunk, seed=16)
    inp = synth.prefill_inputs(1, 160, 2, 128, 128, "bf16", seed=16, device=DEV, with_S0=True, g_const=-5.0,
                               beta_const=1.0)
    _check(inp, chunk=chunk)


@CHUNKS
@pytest.mark.parametrize("io,K,V", [("fp32", 64, 64), ("bf16", 32, 128), ("bf16", 64, 32), ("bf16", 128, 128),
                                     ("fp32", 32, 32)])
def test_passthrough_is_exact(io, K, V, chunk):
    """beta = 0, g = 0: S_final is S0 bit for bit and o_t = S0^T q_t in every chunk
    (the state carried into chunks after the first is checked row by row)."""
    _announce("passthrough", io=io, K=K, V=V, T=150, H=2, chunk=chunk, seed=17)
    inp = synth.prefill_inputs(1, 150, 2, K, V, io, seed=17, device=DEV, with_S0=True, g_const=0.0, beta_const=0.0)
    o, Sf = _run(inp, o_dtype=torch.float32, chunk=chunk)
    assert torch.equal(Sf, inp["S0"])
    o_ref = torch.einsum("bthk,bhkv->bthv", inp["q"].double().cpu(), inp["S0"].double().cpu())
    assert err(o.cpu(), o_ref) <= (TOL_FP32 if io == "fp32" else TOL_BF16)


@CHUNKS
def test_zero_and_one_token(chunk):
    for T in (0, 1):
        _announce("short", T=T, chunk=chunk, seed=18)
        inp = synth.prefill_inputs(1, T, 2, 32, 32, "fp32", seed=18, device=DEV, with_S0=True)
        o, Sf = _run(inp, chunk=chunk)
        if T == 0:
            assert torch.equal(Sf, inp["S0"])
        else:
            _check(inp, io="fp32", chunk=chunk)


@CHUNKS
def test_split_resume_matches_one_call(chunk):
    _announce("split_resume", T=300, chunk=chunk, seed=19)
    inp = synth.prefill_inputs(1, 300, 2, 128, 128, "fp32", seed=19, device=DEV, with_S0=True)
    o, Sf = _run(inp, chunk=chunk)
    s = 123
    a = {n: (x[:, :s].contiguous() if n in ("q", "k", "v", "g", "beta") else x) for n, x in inp.items()}
    oa, Sa = _run(a, chunk=chunk)
    b = {n: (x[:, s:].contiguous() if n in ("q", "k", "v", "g", "beta") else x) for n, x in inp.items()}
    b["S0"] = Sa
    ob, Sb = _run(b, chunk=chunk)
    assert err(torch.cat([oa, ob], 1).cpu(), o.cpu()) <= TOL_FP32
    assert err(Sb.cpu(), Sf.cpu()) <= TOL_FP32


def test_chunk16_and_chunk64_agree():
    """The chunk size is a reformulation: 16- and 64-token chunks give the same result within the
    tolerance, on the benchmark distribution and with mild decay (long carry)."""
    for gs, io in ((0.0, "bf16"), (-6.0, "bf16"), (0.0, "fp32")):
        _announce("chunk16_vs_64", g_shift=gs, io=io, T=777, seed=21)
        inp = synth.prefill_inputs(1, 777, 3, 128, 128, io, seed=21, device=DEV, with_S0=True, g_shift=gs)
        o16, S16 = _run(inp, o_dtype=torch.float32, chunk=16)
        o64, S64 = _run(inp, o_dtype=torch.float32, chunk=64)
        tol = TOL_FP32 if io == "fp32" else TOL_BF16
        assert err(o64.cpu(), o16.cpu()) <= tol and err(S64.cpu(), S16.cpu()) <= tol


@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("K", [32, 64, 128])
@pytest.mark.parametrize("V", [32, 64, 128])
def test_deterministic(io, K, V):
    """Bitwise run-to-run reproducibility (no atomics, no order-dependent reductions),
    over every kernel variant and both chunk sizes; repeats so an intermittent race shows up."""
    _announce("deterministic", io=io, K=K, V=V, seed=20)
    inp = synth.prefill_inputs(1, 500, 4, K, V, io, seed=20, device=DEV, with_S0=True)
    for chunk in (16, 64):
        o1, S1 = _run(inp, o_dtype=torch.float32, chunk=chunk)
        for _ in range(3):
            o2, S2 = _run(inp, o_dtype=torch.float32, chunk=chunk)
            assert torch.equal(o1, o2) and torch.equal(S1, S2), chunk


@CHUNKS
def test_k3_prefill_4k_all_heads(chunk):
    """H=96, T=4096, K=V=128, bf16 (the benchmarked workload, chunk 16 and chunk 64), every head."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("prefill_4k", chunk=chunk, seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp, chunk=chunk)


@CHUNKS
def test_k3_varlen_16_sampled_heads(chunk):
    """16 packed sequences (lengths 256..16384, ~130K tokens), H=96, per-sequence S0;
    the oracle runs on 3 heads, compared with the same heads of the full GPU call."""
    w = synth.WORKLOADS["varlen_16"]
    _announce("varlen_16", chunk=chunk, seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp, heads=(0, 41, 95), chunk=chunk)


SPLIT_CASES = {
    # name: (B, T or lengths, H, K, V, io)
    "single_ragged": (1, 2500, 4, 128, 128, "bf16"),
    "varlen_edges": (1, [0, 700, 1, 1200, 0, 617, 33], 8, 64, 64, "bf16"),
    "batched_fp32": (2, 1100, 3, 32, 128, "fp32"),
}


@pytest.mark.parametrize("operands", ["bf16", "fp16"])
@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_split_calls_are_bit_identical(name, operands):
    """kda_chunk_prep then kda_chunk_state give bitwise what kda_chunk_fwd gives, in either operand format
    (the state pass takes the format from the workspace header the prep wrote), and a second state pass
    over the same prepared workspace gives the same bits again."""
    B, TL, H, K, V, io = SPLIT_CASES[name]
    if io == "fp32" and operands == "fp16":
        pytest.skip("fp16 operands are for bf16 I/O")
    cu = None
    if isinstance(TL, list):
        cu = synth.cu_from_lengths(TL)
        T = cu[-1]
    else:
        T = TL
    _announce("split_calls", case=name, B=B, T=T, H=H, K=K, V=V, io=io, operands=operands, seed=22)
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=22, device=DEV, cu_seqlens=cu, with_S0=True)
    o1, S1 = _run(inp, operands=operands)
    o2, S2, ws = _run_split(inp, operands=operands)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    o3, S3 = chunk_state(inp["v"], ws, K, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(S1, S3)
    assert workspace_status(ws) == 0


def test_varlen_mixed_lengths_against_oracle():
    """Packed sequences of mixed lengths (with an empty one) on 12 heads against the oracle."""
    lengths = [900, 0, 1500, 31, 1100]
    cu = synth.cu_from_lengths(lengths)
    _announce("varlen_mixed", lengths=lengths, H=12, seed=23)
    inp = synth.prefill_inputs(1, cu[-1], 12, 128, 128, "bf16", seed=23, device=DEV, cu_seqlens=cu, with_S0=True)
    _check(inp, heads=(0, 7, 11))


# ------------------------------------------------------------ gate formed in-kernel
#
# With gate="scaled_sigmoid", g holds the gate pre-activation x and kda_chunk_prep forms the
# log-decay -5*sigmoid(x) in fp32 as it reads it; the oracle forms it in fp64 from the same x.

def _gate_inputs(B, T, H, K, V, io, seed, g_scale=1.0, **kw):
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=seed, device=DEV, gate_preact=True, g_scale=g_scale, **kw)
    inp["gate"] = "scaled_sigmoid"
    return inp


@CHUNKS
@pytest.mark.parametrize("io,B,T,H,K,V", [("fp32", 2, 77, 3, 128, 128), ("fp32", 1, 130, 2, 32, 64),
                                          ("bf16", 2, 200, 3, 128, 128), ("bf16", 1, 97, 2, 64, 32)])
def test_gate_fused_shapes(io, B, T, H, K, V, chunk):
    _announce("gate_fused", io=io, B=B, T=T, H=H, K=K, V=V, chunk=chunk, seed=40)
    _check(_gate_inputs(B, T, H, K, V, io, 40, with_S0=True), io=io, chunk=chunk)


@CHUNKS
@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_gate_fused_saturating(io, chunk):
    """x ~ N(0, 30^2): most channels sit at one end of the gate, log-decay ~-5 (the dense-path
    bound) or ~0 (x below about -88, where e^-x overflows fp32 and the gate gives exactly 0)."""
    _announce("gate_saturating", io=io, chunk=chunk, seed=41)
    _check(_gate_inputs(1, 150, 3, 128, 128, io, 41, g_scale=30.0, with_S0=True), io=io, chunk=chunk)


@CHUNKS
def test_gate_fused_varlen(chunk):
    lengths = [37, 0, 16, 1, 150, 64, 0, 65]
    cu = synth.cu_from_lengths(lengths)
    _announce("gate_varlen", lengths=lengths, chunk=chunk, seed=42)
    inp = _gate_inputs(1, cu[-1], 4, 128, 128, "bf16", 42, cu_seqlens=cu, with_S0=True)
    _check(inp, chunk=chunk)


def test_gate_fused_matches_given_log_decay():
    """fp32 I/O: the kernel's in-kernel gate and a log-decay given as input (the oracle's fp64
    gate rounded to fp32) lead to the same outputs, to the fp32 parity bound: the two log-decays
    differ by an ulp or so, which the cumulative sums carry into every decay factor."""
    _announce("gate_vs_given", seed=43)
    inp = _gate_inputs(1, 300, 4, 64, 64, "fp32", 43, with_S0=True)
    o_a, S_a = _run(inp, chunk=16)
    given = dict(inp, g=torch.from_numpy(oracle.scaled_sigmoid_gate(inp["g"].cpu())).float().to(DEV),
                 gate="log_decay")
    o_b, S_b = _run(given, chunk=16)
    res = {"o": err(o_a.cpu(), o_b.cpu()), "S": err(S_a.cpu(), S_b.cpu())}
    print("  differences", res, flush=True)
    assert res["o"] <= TOL_FP32 and res["S"] <= TOL_FP32, res


def test_gate_fused_k3_prefill_4k_sampled_heads():
    """The gate-fused leg of the benchmark: H=96, T=4096, K=V=128, bf16, chunk 16, g = x ~ N(0,1)
    pre-activations; the oracle runs on 4 heads of the full GPU call."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("gate_prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV, gate_preact=True)
    inp["gate"] = "scaled_sigmoid"
    _check(inp, heads=(0, 31, 64, 95))


# ------------------------------------------------------------ output gate
#
# With o_gate given, the state pass's o store multiplies by sigmoid(o_gate) in fp32; the oracle
# applies the same gate in fp64 to its output.

@CHUNKS
@pytest.mark.parametrize("io,B,T,H,K,V", [("fp32", 2, 77, 3, 128, 128), ("fp32", 1, 50, 2, 64, 32),
                                          ("bf16", 2, 200, 3, 128, 128), ("bf16", 1, 129, 2, 128, 64)])
def test_output_gate_shapes(io, B, T, H, K, V, chunk):
    _announce("output_gate", io=io, B=B, T=T, H=H, K=K, V=V, chunk=chunk, seed=50)
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=50, device=DEV, with_S0=True, with_o_gate=True)
    _check(inp, io=io, chunk=chunk)


@CHUNKS
def test_output_gate_varlen_both_gates(chunk):
    """Packed sequences (empty and ragged ones) with both gates formed in-kernel."""
    lengths = [37, 0, 16, 1, 150, 64, 0, 65]
    cu = synth.cu_from_lengths(lengths)
    _announce("both_gates_varlen", lengths=lengths, chunk=chunk, seed=51)
    inp = _gate_inputs(1, cu[-1], 4, 128, 128, "bf16", 51, cu_seqlens=cu, with_S0=True, with_o_gate=True)
    _check(inp, chunk=chunk)


def test_output_gate_leaves_state_and_scales_o():
    """fp32 I/O: the gate changes o only: S_final is bitwise that of the ungated call, and z = 0 halves o
    (sigmoid(0) = 1/2 exactly, a power-of-two scale)."""
    _announce("output_gate_exact", seed=52)
    inp = synth.prefill_inputs(1, 300, 4, 64, 64, "fp32", seed=52, device=DEV, with_S0=True)
    o1, S1 = _run(inp)
    o2, S2 = _run(dict(inp, o_gate=torch.zeros_like(inp["v"])))
    assert torch.equal(S1, S2) and torch.equal(o2, 0.5 * o1)


@pytest.mark.parametrize("operands", ["bf16", "fp16"])
def test_output_gate_split_calls(operands):
    """The split calls apply the output gate as kda_chunk_fwd does (bitwise), in either operand format."""
    _announce("output_gate_split", operands=operands, seed=53)
    inp = synth.prefill_inputs(1, 2500, 4, 128, 128, "bf16", seed=53, device=DEV, with_S0=True, with_o_gate=True)
    o1, S1 = _run(inp, operands=operands)
    o2, S2, _ = _run_split(inp, operands=operands)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    _check(inp, heads=(0, 3), operands=operands)


def test_output_gate_k3_prefill_4k_sampled_heads():
    """The both-gates leg of the benchmark: H=96, T=4096, K=V=128, bf16, chunk 16; 4 heads checked."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("both_gates_prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV, gate_preact=True, with_o_gate=True)
    inp["gate"] = "scaled_sigmoid"
    _check(inp, heads=(0, 31, 64, 95))


# ------------------------------------------------------------ q/k L2 normalisation in-kernel
#
# With qk_norm, the prep kernels divide each raw q and k row (per token and head) by
# sqrt(|x|^2 + 1e-6) in fp32 as they read it; the oracle normalises the same raw rows in fp64.

def _norm_inputs(B, T, H, K, V, io, seed, **kw):
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=seed, device=DEV, raw_k=True, **kw)
    inp["qk_norm"] = True
    return inp


@CHUNKS
@pytest.mark.parametrize("io,B,T,H,K,V", [("fp32", 2, 77, 3, 128, 128), ("fp32", 1, 130, 2, 32, 64),
                                          ("bf16", 2, 200, 3, 128, 128), ("bf16", 1, 97, 2, 64, 32)])
def test_qk_norm_shapes(io, B, T, H, K, V, chunk):
    _announce("qk_norm", io=io, B=B, T=T, H=H, K=K, V=V, chunk=chunk, seed=60)
    _check(_norm_inputs(B, T, H, K, V, io, 60, with_S0=True), io=io, chunk=chunk)


@CHUNKS
def test_qk_norm_varlen_with_both_gates(chunk):
    """Packed sequences (empty and ragged ones), raw q and k normalised in-kernel, both gates formed
    in-kernel: the whole prologue and epilogue at once."""
    lengths = [37, 0, 16, 1, 150, 64, 0, 65]
    cu = synth.cu_from_lengths(lengths)
    _announce("qk_norm_varlen_gates", lengths=lengths, chunk=chunk, seed=61)
    inp = _norm_inputs(1, cu[-1], 4, 128, 128, "bf16", 61, cu_seqlens=cu, with_S0=True, gate_preact=True,
                       with_o_gate=True)
    inp["gate"] = "scaled_sigmoid"
    _check(inp, chunk=chunk)


def test_qk_norm_zero_and_tiny_rows():
    """fp32: all-zero q and k rows stay zero (no NaN: the 1e-6 under the root), and rows scaled by
    1e-3 are still normalised (their |x|^2 ~ 1e-4 is well above 1e-6)."""
    _announce("qk_norm_zero_rows", seed=62)
    inp = _norm_inputs(1, 70, 2, 64, 64, "fp32", 62, with_S0=True)
    inp["q"][0, 5] = 0.0
    inp["k"][0, 9] = 0.0
    inp["k"][0, 20:40] *= 1e-3
    inp["q"][0, 30:50] *= 1e-3
    for chunk in (16, 64):
        o, Sf = _check(inp, io="fp32", chunk=chunk)
        assert torch.isfinite(o).all() and torch.isfinite(Sf).all()


def test_qk_norm_matches_host_normalised():
    """fp32: normalising raw rows in the kernel and passing rows normalised on the host (the oracle's
    fp64 normalisation rounded to fp32) agree to the fp32 parity bound, through prefill and decode."""
    _announce("qk_norm_vs_host", seed=63)
    inp = _norm_inputs(1, 300, 4, 64, 64, "fp32", 63, with_S0=True)
    o_a, S_a = _run(inp, chunk=16)
    host = dict(inp, q=torch.from_numpy(oracle.l2_normalize(inp["q"].cpu())).float().to(DEV),
                k=torch.from_numpy(oracle.l2_normalize(inp["k"].cpu())).float().to(DEV), qk_norm=False)
    o_b, S_b = _run(host, chunk=16)
    res = {"o": err(o_a.cpu(), o_b.cpu()), "S": err(S_a.cpu(), S_b.cpu())}
    print("  differences", res, flush=True)
    assert res["o"] <= TOL_FP32 and res["S"] <= TOL_FP32, res


@pytest.mark.parametrize("operands", ["bf16", "fp16"])
def test_qk_norm_split_calls(operands):
    """The split calls normalise as kda_chunk_fwd does (bitwise), in either operand format."""
    _announce("qk_norm_split", operands=operands, seed=64)
    inp = _norm_inputs(1, 2500, 4, 128, 128, "bf16", 64, with_S0=True, with_o_gate=True)
    o1, S1 = _run(inp, operands=operands)
    o2, S2, _ = _run_split(inp, operands=operands)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    _check(inp, heads=(0, 3), operands=operands)


def test_all_fused_k3_prefill_4k_sampled_heads():
    """The prologue-and-epilogue leg of the benchmark: H=96, T=4096, K=V=128, bf16, chunk 16, raw q
    and k normalised in-kernel, both gates formed in-kernel; 4 heads checked."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("all_fused_prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV, gate_preact=True, with_o_gate=True, raw_k=True)
    inp["gate"] = "scaled_sigmoid"
    inp["qk_norm"] = True
    _check(inp, heads=(0, 31, 64, 95))


# ------------------------------------------------------------ short convolution in-kernel
#
# With conv, the prep kernels convolve the raw q and k rows (length 4, causal, per channel, zero history
# at each sequence start, optional SiLU) as they read them, and kda_conv_v convolves v into the workspace
# for the state pass; the oracle convolves the same raw rows in fp64.

def _conv_taps(H, K, V, seed):
    g = torch.Generator().manual_seed(seed)
    return (0.5 * torch.randn((H, 2 * K + V, 4), generator=g)).to(DEV)


def _conv_inputs(B, T, H, K, V, io, seed, conv="short4_silu", **kw):
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=seed, device=DEV, **kw)
    inp["conv"] = conv
    inp["conv_w"] = _conv_taps(H, K, V, seed)
    return inp


@CHUNKS
@pytest.mark.parametrize("io,B,T,H,K,V,conv", [("fp32", 2, 77, 3, 128, 128, "short4"),
                                               ("fp32", 1, 130, 2, 32, 64, "short4_silu"),
                                               ("bf16", 2, 200, 3, 128, 128, "short4_silu"),
                                               ("bf16", 1, 97, 2, 64, 32, "short4")])
def test_conv_shapes(io, B, T, H, K, V, conv, chunk):
    _announce("conv", io=io, B=B, T=T, H=H, K=K, V=V, conv=conv, chunk=chunk, seed=70)
    _check(_conv_inputs(B, T, H, K, V, io, 70, conv=conv, with_S0=True), io=io, chunk=chunk)


@CHUNKS
def test_conv_varlen_whole_prologue(chunk):
    """Packed sequences (empty, 1- and 2-token ones: the history restarts inside a chunk), convolution with
    SiLU, q/k normalisation and both gates at once."""
    lengths = [37, 0, 2, 1, 150, 64, 0, 65, 3]
    cu = synth.cu_from_lengths(lengths)
    _announce("conv_varlen", lengths=lengths, chunk=chunk, seed=71)
    inp = _conv_inputs(1, cu[-1], 4, 128, 128, "bf16", 71, cu_seqlens=cu, with_S0=True, gate_preact=True,
                       with_o_gate=True, raw_k=True)
    inp["gate"] = "scaled_sigmoid"
    inp["qk_norm"] = True
    _check(inp, chunk=chunk)


def test_conv_identity_taps_change_nothing():
    """Taps (0, 0, 0, 1) without SiLU give every input back exactly, so o and S_final equal those of the call
    without a convolution bit for bit where both calls carry the same operand format (fp32; bf16 at 64-token
    chunks). At 16-token chunks a bf16 call without a convolution carries the state pass's operands as fp16
    and one with a convolution as bf16 hi + lo pairs: there the two agree to the parity bound."""
    _announce("conv_identity", seed=72)
    for io in ("fp32", "bf16"):
        inp = synth.prefill_inputs(2, 90, 3, 64, 128, io, seed=72, device=DEV, with_S0=True)
        w = torch.zeros((3, 2 * 64 + 128, 4), device=DEV)
        w[..., 3] = 1.0
        for chunk in (16, 64):
            o1, S1 = _run(inp, chunk=chunk)
            o2, S2 = _run(dict(inp, conv="short4", conv_w=w), chunk=chunk)
            if io == "bf16" and chunk == 16:
                o1f, _ = _run(inp, chunk=chunk, o_dtype=torch.float32)
                o2f, _ = _run(dict(inp, conv="short4", conv_w=w), chunk=chunk, o_dtype=torch.float32)
                assert err(o1f.cpu(), o2f.cpu()) <= TOL_BF16 and err(S1.cpu(), S2.cpu()) <= TOL_BF16
            else:
                assert torch.equal(o1, o2) and torch.equal(S1, S2), (io, chunk)


def test_conv_split_calls_match_one_call():
    """kda_chunk_prep then kda_chunk_state with a convolution give bitwise what kda_chunk_fwd gives."""
    _announce("conv_split", seed=73)
    B, T, H, K, V = 1, 300, 4, 128, 128
    inp = _conv_inputs(B, T, H, K, V, "bf16", 73, with_S0=True)
    o1, S1 = _run(inp)
    o2, S2, _ = _run_split(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_conv_k3_prefill_4k_sampled_heads():
    """The convolution leg of the benchmark: H=96, T=4096, K=V=128, bf16, chunk 16, raw q and k, SiLU
    convolution, normalisation and both gates in-kernel; 4 heads checked."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("conv_prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV, gate_preact=True, with_o_gate=True, raw_k=True)
    inp["gate"] = "scaled_sigmoid"
    inp["qk_norm"] = True
    inp["conv"] = "short4_silu"
    g = torch.Generator().manual_seed(7)
    inp["conv_w"] = (0.5 * torch.randn((w.H, 2 * w.K + w.V, 4), generator=g)).to(DEV)
    _check(inp, heads=(0, 31, 64, 95))


@pytest.mark.parametrize("chunk", [16, 64])
def test_conv_path_deterministic(chunk):
    """The convolution variants (kda_conv_x, the conv prep, the hi + lo state pass) with the whole prologue
    and epilogue give bitwise the same o and S_final on every call."""
    _announce("conv_deterministic", chunk=chunk, seed=74)
    lengths = [200, 3, 0, 77]
    cu = synth.cu_from_lengths(lengths)
    inp = _conv_inputs(1, cu[-1], 3, 128, 128, "bf16", 74, cu_seqlens=cu, with_S0=True, gate_preact=True,
                       with_o_gate=True, raw_k=True)
    inp["gate"] = "scaled_sigmoid"
    inp["qk_norm"] = True
    o1, S1 = _run(inp, chunk=chunk)
    for _ in range(3):
        o2, S2 = _run(inp, chunk=chunk)
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ------------------------------------------------------------ operand formats at 16-token chunks
#
# bf16 I/O at 16-token chunks takes the state pass's operands as bf16 hi + lo pairs by default
# (bf16's range); operands="fp16" selects fp16 operands (fewer bytes and products, fp16's range).


def test_fp16_operands_k3_prefill_4k_all_heads():
    """The fp16 operand format on the 4096-token workload, every head, and the split calls' workspace query
    (smaller than the bf16 pairs')."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("k3_prefill_4k_fp16_operands", seed=w.seed)
    nbf = prep_workspace_bytes(1, w.T, w.H, w.K, w.V, 1, 16, "bf16")
    n16 = prep_workspace_bytes(1, w.T, w.H, w.K, w.V, 1, 16, "bf16", operands="fp16")
    assert 0 < n16 < nbf
    inp = synth.workload_prefill_inputs(w, device=DEV)
    _check(inp, operands="fp16")


@pytest.mark.parametrize("scale", [1e3, 3e4, 1e5])
def test_large_values_default_operands(scale):
    """bf16 inputs far outside the normalised range: v and S0 scaled by up to 1e5 (beyond fp16's largest
    value, 65504). The default bf16-pair operands keep bf16's exponent range, so the call still meets the
    bf16 bound against the oracle."""
    _announce("large_values", scale=scale, seed=76)
    lengths = [300, 17, 0, 190]
    cu = synth.cu_from_lengths(lengths)
    inp = synth.prefill_inputs(1, cu[-1], 3, 128, 128, "bf16", seed=76, device=DEV, cu_seqlens=cu, with_S0=True)
    inp["v"] = (inp["v"].float() * scale).to(torch.bfloat16)
    inp["S0"] = inp["S0"] * scale
    _check(inp)


def test_large_values_fp16_operands_are_not_finite():
    """The documented limit of the fp16 format: with |v| beyond 65504 the results are not finite (they never
    come out as wrong finite numbers); the default format on the same inputs is finite and in bound."""
    _announce("large_values_fp16", seed=77)
    inp = synth.prefill_inputs(1, 200, 2, 128, 128, "bf16", seed=77, device=DEV, with_S0=True)
    inp["v"] = (inp["v"].float() * 1e5).to(torch.bfloat16)
    o, Sf = _run(inp, operands="fp16", o_dtype=torch.float32)
    assert not bool(torch.isfinite(o).all()) and not bool(torch.isfinite(Sf).all())
    o2, S2 = _run(inp, o_dtype=torch.float32)
    assert bool(torch.isfinite(o2).all()) and bool(torch.isfinite(S2).all())


def test_state_refuses_a_workspace_of_another_call():
    """kda_chunk_state over a workspace that kda_chunk_prep filled for other sizes, or that no prep filled,
    reads none of it: o and S_final come out NaN and the header's error word says why."""
    _announce("workspace_header_mismatch", seed=78)
    inp = synth.prefill_inputs(1, 300, 4, 64, 64, "bf16", seed=78, device=DEV, with_S0=True)
    _, _, ws = _run_split(inp)
    short = synth.prefill_inputs(1, 200, 4, 64, 64, "bf16", seed=78, device=DEV, with_S0=True)
    o = torch.zeros((1, 200, 4, 64), dtype=torch.bfloat16, device=DEV)
    Sf = torch.zeros((1, 4, 64, 64), dtype=torch.float32, device=DEV)
    chunk_state(short["v"], ws, 64, S0=short["S0"], out=o, final_state_out=Sf)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o.float()).all()) and bool(torch.isnan(Sf).all())
    assert workspace_status(ws) == _lib.WS_ERR_HEADER_MISMATCH
    # the workspace of a fused (low-memory) kda_chunk_fwd holds no factors, and its header says so: the
    # call runs on the leading min_workspace_bytes of a buffer as large as the two passes need, and the
    # state pass is then handed the whole buffer (its size passes the host check; the header does not)
    wsf = torch.full((prep_workspace_bytes(1, 300, 4, 64, 64, 1, 16, "bf16"),), 0xFF, dtype=torch.uint8, device=DEV)
    chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S0=inp["S0"],
              workspace=wsf[:min_workspace_bytes(1, 300, 4, 64, 64, 1, 16, "bf16")])
    o3 = torch.zeros((1, 300, 4, 64), dtype=torch.bfloat16, device=DEV)
    chunk_state(inp["v"], wsf, 64, S0=inp["S0"], out=o3, final_state_out=Sf)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o3.float()).all()) and bool(torch.isnan(Sf).all())
    assert workspace_status(wsf) == _lib.WS_ERR_HEADER_MISMATCH
    # a workspace no prep has written: its header has no magic, the outputs are NaN all the same
    ws2 = torch.zeros_like(ws)
    o.zero_()
    Sf.zero_()
    chunk_state(inp["v"][:, :200].contiguous(), ws2, 64, S0=inp["S0"], out=o, final_state_out=Sf)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o.float()).all()) and bool(torch.isnan(Sf).all())


# ------------------------------------------------------------ the low-memory (fused) form
#
# With less workspace than the two passes need (but at least min_workspace_bytes), kda_chunk_fwd runs one
# kernel whose prep wavefronts form each sub-tile's factors straight into the state pass's LDS ring: the
# same arithmetic as kda_chunk_prep + kda_chunk_state, so the same bits.

LOWMEM_CASES = {
    "batched_ragged": (2, 200, 3, 128, 128, "bf16", None),
    "varlen_edges": (1, [37, 0, 16, 1, 150, 64, 0, 65], 4, 64, 64, "bf16", None),
    "small_dims": (1, 130, 2, 32, 128, "bf16", None),
    "fp32": (2, 77, 3, 128, 64, "fp32", None),
}


@pytest.mark.parametrize("operands", ["bf16", "fp16"])
@pytest.mark.parametrize("name", list(LOWMEM_CASES))
def test_low_memory_form_is_bit_identical_and_in_bound(name, operands):
    B, TL, H, K, V, io, _ = LOWMEM_CASES[name]
    if io == "fp32" and operands == "fp16":
        pytest.skip("fp16 operands are for bf16 I/O")
    cu = None
    if isinstance(TL, list):
        cu = synth.cu_from_lengths(TL)
        T = cu[-1]
    else:
        T = TL
    _announce("low_memory", case=name, B=B, T=T, H=H, K=K, V=V, io=io, operands=operands, seed=81)
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed=81, device=DEV, cu_seqlens=cu, with_S0=True)
    o1, S1 = _run(inp, operands=operands)
    o2, S2 = _run_low_memory(inp, operands=operands)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_low_memory_form_with_gates_and_norm():
    """Both gates and the q/k normalisation through the fused form: bitwise the two-pass result."""
    _announce("low_memory_prologue", seed=82)
    inp = _norm_inputs(1, 700, 4, 128, 128, "bf16", 82, with_S0=True, with_o_gate=True)
    o1, S1 = _run(inp)
    o2, S2 = _run_low_memory(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_low_memory_form_k3_prefill_4k_all_heads():
    """The 4096-token, 96-head workload through the fused form against the oracle (every head)."""
    w = synth.WORKLOADS["prefill_4k"]
    _announce("low_memory_prefill_4k", seed=w.seed)
    inp = synth.workload_prefill_inputs(w, device=DEV)
    o_ref, S_ref = _oracle(inp)
    o, Sf = _run_low_memory(inp, o_dtype=torch.float32)
    res = {"o_fp32": err(o.cpu(), o_ref), "S": err(Sf.cpu(), S_ref)}
    print("  errors", res, flush=True)
    assert res["o_fp32"] <= TOL_BF16 and res["S"] <= TOL_BF16, res
