"""GPU parity of kda_chunk_bwd (through the C ABI) against the fp64 backward oracle.

The backward runs in fp32 on inputs the oracle sees exactly (bf16 or fp32, widened to fp64), and its
outputs are fp32, so every gradient is held to the fp32 bound of the forward, err <= 1e-4 (max abs
difference over the rms of the reference), for both I/O dtypes.
"""
import numpy as np
import pytest
import torch

import oracle
from kda_gated_delta_chunk_amd import _lib, chunk_bwd, chunk_fwd
from kda_gated_delta_chunk_amd import synth
from tests.parity import TOL_FP32, err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0", "do_gate", "dconv_w")


def _announce(name, **kw):
    print("\n[case] %s %s" % (name, " ".join("%s=%s" % kv for kv in kw.items())), flush=True)


def _inputs(B, T, H, K, V, io, seed, cu=None, with_S0=True, with_dsf=True, **kw):
    inp = synth.prefill_inputs(B, T, H, K, V, io, seed, DEV, cu_seqlens=cu, with_S0=with_S0, **kw)
    N = B if cu is None else len(cu) - 1
    do, dsf = synth.output_grads(B, T, H, V, io, seed, DEV, num_seqs=N, K=K)
    inp["do"] = do
    inp["dS_final"] = dsf if with_dsf else None
    return inp


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def _gpu(inp, want_dS0=True, seg=0):
    """The GPU gradients, written over NaN-filled outputs and a NaN-filled workspace (so an element the kernels
    leave unwritten, or a workspace byte read before it is written, shows up in the comparison). seg > 0: a
    workspace of the size for segments of seg tokens, so the call takes the input in segments."""
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    out = {"dq": _nan((B, T, H, K)), "dk": _nan((B, T, H, K)), "dg": _nan((B, T, H, K)), "dv": _nan((B, T, H, V)),
           "dbeta": _nan((B, T, H))}
    if want_dS0:
        out["dS0"] = _nan((N, H, K, V))
    if inp.get("o_gate") is not None:
        out["do_gate"] = _nan((B, T, H, V))
    if inp.get("conv", "none") != "none":
        out["dconv_w"] = _nan((H, 2 * K + V, 4))
    qc = _lib.KDA_QK_L2NORM if inp.get("qk_norm", False) else _lib.KDA_QK_AS_GIVEN
    cc = _lib.CONVS[inp.get("conv", "none")]
    if seg:
        wsb = _lib.load().kda_chunk_bwd_segmented_workspace_bytes(B, T, H, K, V, N, qc, cc, seg)
        assert 0 < wsb < _lib.load().kda_chunk_bwd_workspace_bytes(B, T, H, K, V, N, qc, cc)
    else:
        wsb = _lib.load().kda_chunk_bwd_workspace_bytes(B, T, H, K, V, N, qc, cc)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN patterns in every fp32 word
    got = chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"], S0=inp["S0"],
                    dS_final=inp["dS_final"], cu_seqlens=inp["cu_seqlens"], want_dS0=want_dS0,
                    gate=inp.get("gate", "log_decay"), o_gate=inp.get("o_gate"), qk_norm=inp.get("qk_norm", False),
                    conv=inp.get("conv", "none"), conv_w=inp.get("conv_w"), workspace=ws, out=out)
    torch.cuda.synchronize()
    for name in out:
        assert got[name] is out[name], name
    return got


def _oracle(inp, heads=None):
    names = ("q", "k", "v", "g", "beta", "do")
    xs = [inp[n] for n in names]
    z = inp.get("o_gate")
    if z is not None and heads is not None:
        z = z[:, :, list(heads)]
    S0, dsf = inp["S0"], inp["dS_final"]
    if heads is not None:
        hs = list(heads)
        xs = [x[:, :, hs] for x in xs]
        S0 = None if S0 is None else S0[:, hs]
        dsf = None if dsf is None else dsf[:, hs]
    cu = inp["cu_seqlens"]
    cw = inp.get("conv_w")
    if cw is not None and heads is not None:
        cw = cw[list(heads)]
    return oracle.chunk_bwd(*(x.cpu() for x in xs), S0=None if S0 is None else S0.cpu(),
                            dS_final=None if dsf is None else dsf.cpu(), cu_seqlens=None if cu is None else cu.cpu(),
                            gate=inp.get("gate", "log_decay"), o_gate=None if z is None else z.cpu(),
                            qk_norm=inp.get("qk_norm", False), conv=inp.get("conv", "none"),
                            conv_w=None if cw is None else cw.cpu())


def _compare(out, ref, heads=None, tol=TOL_FP32):
    errs = {}
    for n in NAMES:
        if n not in out:
            continue
        x = out[n]
        if heads is not None:
            if n == "dconv_w":
                x = x[list(heads)]
            elif n == "dS0":
                x = x[:, list(heads)]
            else:
                x = x[:, :, list(heads)]
        assert n in ref, n
        errs[n] = err(x, ref[n])
    print("  errors " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= tol, (n, e)
    return errs


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", [
    # (B, T, H, K, V)
    (1, 64, 2, 32, 32),
    (2, 37, 3, 64, 64),      # ragged tail segment, two batch rows
    (1, 50, 2, 128, 128),
    (1, 9, 1, 128, 32),
    (3, 1, 2, 32, 128),      # one token per sequence
])
def test_bwd_matches_oracle(io, shape):
    B, T, H, K, V = shape
    _announce("bwd", io=io, B=B, T=T, H=H, K=K, V=V, seed=71)
    inp = _inputs(B, T, H, K, V, io, 71)
    _compare(_gpu(inp), _oracle(inp))


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_varlen_with_an_empty_sequence(io):
    cu = [0, 5, 5, 40, 77, 93]
    _announce("bwd_varlen", io=io, cu=cu, H=3, K=64, V=128, seed=72)
    inp = _inputs(1, cu[-1], 3, 64, 128, io, 72, cu=cu)
    _compare(_gpu(inp), _oracle(inp))


def test_bwd_without_S0_dS_final_or_dS0():
    _announce("bwd_optional", H=2, K=64, V=64, T=40, seed=73)
    inp = _inputs(1, 40, 2, 64, 64, "fp32", 73, with_S0=False, with_dsf=False)
    out = _gpu(inp, want_dS0=False)
    assert "dS0" not in out
    _compare(out, _oracle(inp))


def test_bwd_empty_batch_passes_dS_final_through():
    _announce("bwd_empty", T=0, H=2, K=32, V=32)
    inp = _inputs(1, 0, 2, 32, 32, "fp32", 74)
    out = _gpu(inp)
    assert torch.equal(out["dS0"], inp["dS_final"])
    assert out["dq"].numel() == 0


def test_bwd_mild_decay_long_carry():
    # g = -5 sigmoid(x - 6): retention ~0.988, so gradients carry across hundreds of tokens
    _announce("bwd_mild", T=300, H=2, K=128, V=128, seed=75)
    inp = _inputs(1, 300, 2, 128, 128, "fp32", 75, g_shift=-6.0)
    _compare(_gpu(inp), _oracle(inp))


def test_bwd_segments_chained_through_the_states():
    # A long sequence backpropagated in segments: the forward of the first segment gives the state entering the
    # second; the second's backward gives dL/d(that state), which is the first segment's dL/dS_final. The
    # chained gradients equal one call's (to fp32 rounding), with workspace bounded by the segment length.
    _announce("bwd_segments", T=1000, split=392, H=3, K=128, V=128, seed=77)
    inp = _inputs(1, 1000, 3, 128, 128, "fp32", 77, g_shift=-6.0)
    whole = _gpu(inp)
    T1 = 392

    def part(a, b):
        seg = {n: inp[n][:, a:b].contiguous() for n in ("q", "k", "v", "g", "beta", "do")}
        seg["cu_seqlens"] = None
        return seg

    _, S_mid = chunk_fwd(*(inp[n][:, :T1].contiguous() for n in ("q", "k", "v", "g", "beta")), S0=inp["S0"])
    second = part(T1, 1000)
    second["S0"], second["dS_final"] = S_mid, inp["dS_final"]
    g2 = _gpu(second)
    first = part(0, T1)
    first["S0"], first["dS_final"] = inp["S0"], g2["dS0"]
    g1 = _gpu(first)
    errs = {n: err(torch.cat([g1[n], g2[n]], dim=1), whole[n]) for n in ("dq", "dk", "dv", "dg", "dbeta")}
    errs["dS0"] = err(g1["dS0"], whole["dS0"])
    print("  errors " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n, e in errs.items():
        assert e <= TOL_FP32, (n, e)


def _same(got, ref):
    # In segments the gradients are bitwise one call's: every segment of a sequence holds an even number of
    # 16-token chunks, so each chunk keeps its place in its pair (which state the gradient kernel stores and
    # which it rebuilds), and the state crosses a segment boundary in fp32 as it crosses a chunk boundary.
    errs = {n: err(got[n], ref[n]) for n in ref}
    print("  against one call " + " ".join("%s=%.2e" % kv for kv in errs.items()), flush=True)
    for n in ref:
        assert torch.equal(got[n], ref[n]), (n, errs[n])


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_in_segments_matches_one_call(io):
    # a workspace for 128-token segments: the 1000-token sequence runs as 8 segments chained through their
    # states (mild decay, so the state carries across several segments); the same gradients as one call
    _announce("bwd_in_segments", io=io, T=1000, H=3, K=64, V=64, seg=128, seed=81)
    inp = _inputs(1, 1000, 3, 64, 64, io, 81, g_shift=-6.0)
    got = _gpu(inp, seg=128)
    _same(got, _gpu(inp))
    _compare(got, _oracle(inp))


def test_bwd_in_segments_varlen_with_the_prologue_and_gates():
    # packed sequences of 5, 0, 295, 1, 399 and 300 tokens with 64-token segments: the short ones share calls,
    # the long ones are chained; q/k normalisation, the gate pre-activation and the output gate
    cu = [0, 5, 5, 300, 301, 700, 1000]
    _announce("bwd_in_segments_varlen", cu=cu, H=2, K=128, V=64, io="bf16", seg=64, seed=82)
    inp = _inputs(1, 1000, 2, 128, 64, "bf16", 82, cu=cu, gate_preact=True, with_o_gate=True)
    inp["gate"] = "scaled_sigmoid"
    inp["qk_norm"] = True
    got = _gpu(inp, seg=64)
    _same(got, _gpu(inp))
    _compare(got, _oracle(inp))


@pytest.mark.parametrize("B,T,seg", [(4, 40, 96), (2, 150, 64)])
def test_bwd_in_segments_batched_rows(B, T, seg):
    # batched rows: two 40-token rows per call (B=4, 96-token segments), or each 150-token row in 3 segments
    _announce("bwd_in_segments_rows", B=B, T=T, H=2, K=32, V=32, seg=seg, seed=83)
    inp = _inputs(B, T, 2, 32, 32, "fp32", 83)
    got = _gpu(inp, seg=seg)
    _same(got, _gpu(inp))
    _compare(got, _oracle(inp))


def test_bwd_4k_workload_in_segments():
    # the 4096-token, 96-head bf16 workload with a workspace under 1 GB (segments of at most 1024 tokens),
    # against one call on every head
    _announce("bwd_4k_in_segments", T=4096, H=96, K=128, V=128, io="bf16", seg=1024, seed=1002)
    inp = _inputs(1, 4096, 96, 128, 128, "bf16", 1002, with_S0=False)
    wsb = _lib.load().kda_chunk_bwd_segmented_workspace_bytes(1, 4096, 96, 128, 128, 1, 0, 0, 1024)
    assert wsb < 1 << 30
    _same(_gpu(inp, seg=1024), _gpu(inp))


def test_bwd_1m_tokens_in_segments():
    # the million-token context: two heads of one 1,048,576-token sequence, in 65,536-token segments (a
    # workspace of 1.3 GB instead of 18 GB), against one call
    T, H = 1 << 20, 2
    _announce("bwd_1m_in_segments", T=T, H=H, K=128, V=128, io="bf16", seg=65536, seed=1003)
    inp = _inputs(1, T, H, 128, 128, "bf16", 1003)
    got = _gpu(inp, seg=65536)
    for n in got:
        assert torch.isfinite(got[n]).all(), n
    _same(got, _gpu(inp))


def test_bwd_is_deterministic():
    _announce("bwd_determinism", T=200, H=4, K=128, V=128, seed=76)
    inp = _inputs(1, 200, 4, 128, 128, "bf16", 76)
    a, b = _gpu(inp), _gpu(inp)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_bwd_4k_workload_sampled_heads():
    # the 4096-token, 96-head bf16 workload of the prefill benchmark, in one call; heads 0 and 95 end to end
    _announce("bwd_4k", T=4096, H=96, K=128, V=128, io="bf16", seed=1001)
    inp = _inputs(1, 4096, 96, 128, 128, "bf16", 1001, with_S0=False)
    out = _gpu(inp)
    for n in out:
        assert torch.isfinite(out[n]).all(), n
    heads = (0, 95)
    _compare(out, _oracle(inp, heads), heads)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_gate_preactivation(io):
    # g holds the gate pre-activation x ~ 2 N(0, 1); the kernels form -5 sigmoid(x) and return dL/dx
    _announce("bwd_gate", io=io, T=70, H=3, K=128, V=64, seed=77)
    inp = _inputs(1, 70, 3, 128, 64, io, 77, gate_preact=True, g_scale=2.0)
    inp["gate"] = "scaled_sigmoid"
    _compare(_gpu(inp), _oracle(inp))


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_output_gate_and_gate_preactivation(io):
    # both gates of the forward: g is the pre-activation x, and o = core output * sigmoid(z); dL/dz is returned
    _announce("bwd_gates", io=io, T=53, H=2, K=64, V=128, seed=78)
    inp = _inputs(1, 53, 2, 64, 128, io, 78, gate_preact=True, with_o_gate=True)
    inp["gate"] = "scaled_sigmoid"
    out = _gpu(inp)
    assert "do_gate" in out
    _compare(out, _oracle(inp))


# ------------------------------------------------------------ through the prologue
#
# The forward's q/k normalisation and short convolution (length 4, causal, restarting at each sequence
# start, optional SiLU) are taken back by the chain rule: dq, dk and dv are with respect to the raw inputs,
# and dconv_w is the gradient of the taps. The oracle runs the same prologue in fp64.

def _taps(H, K, V, seed, scale=0.5):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn((H, 2 * K + V, 4), generator=g)).to(DEV)


def _prologue(inp, qk_norm, conv, seed):
    inp["qk_norm"] = qk_norm
    inp["conv"] = conv
    if conv != "none":
        H, K, V = inp["q"].shape[2], inp["q"].shape[3], inp["v"].shape[3]
        inp["conv_w"] = _taps(H, K, V, seed)
    return inp


PROLOGUES = [(True, "none"), (False, "short4"), (False, "short4_silu"), (True, "short4_silu")]


@pytest.mark.parametrize("io", ["fp32", "bf16"])
@pytest.mark.parametrize("qk_norm,conv", PROLOGUES)
def test_bwd_prologue_matches_oracle(io, qk_norm, conv):
    # two batch rows of 150 tokens: several 64-token tiles of the taps' partial sums and a ragged tail
    _announce("bwd_prologue", io=io, qk_norm=qk_norm, conv=conv, B=2, T=150, H=3, K=64, V=128, seed=81)
    inp = _prologue(_inputs(2, 150, 3, 64, 128, io, 81, raw_k=qk_norm), qk_norm, conv, 81)
    out = _gpu(inp)
    assert ("dconv_w" in out) == (conv != "none")
    _compare(out, _oracle(inp))


@pytest.mark.parametrize("K,V", [(32, 32), (128, 128), (128, 64)])
def test_bwd_prologue_head_sizes(K, V):
    _announce("bwd_prologue_sizes", K=K, V=V, T=70, H=2, seed=82)
    inp = _prologue(_inputs(1, 70, 2, K, V, "bf16", 82, raw_k=True), True, "short4_silu", 82)
    _compare(_gpu(inp), _oracle(inp))


def test_bwd_prologue_varlen_and_both_gates():
    """Packed sequences (empty, 1- and 2-token ones, so the convolution's history restarts inside a 64-token
    tile and a tile's window crosses sequence ends), both gates, the normalisation and SiLU at once."""
    lengths = [37, 0, 2, 1, 150, 64, 0, 65, 3]
    cu = synth.cu_from_lengths(lengths)
    _announce("bwd_prologue_varlen", lengths=lengths, H=2, K=128, V=64, seed=83)
    inp = _inputs(1, cu[-1], 2, 128, 64, "bf16", 83, cu=cu, gate_preact=True, with_o_gate=True, raw_k=True)
    inp["gate"] = "scaled_sigmoid"
    inp = _prologue(inp, True, "short4_silu", 83)
    out = _gpu(inp)
    assert "do_gate" in out and "dconv_w" in out
    _compare(out, _oracle(inp))


def test_bwd_prologue_packed_rows_past_the_last_sequence():
    # cu_seqlens ends before B * T: rows past it are read by no sequence; their gradients are not written
    cu = [0, 30, 61]
    _announce("bwd_prologue_tail", cu=cu, T=100, H=2, K=64, V=64, seed=84)
    inp = _inputs(1, 100, 2, 64, 64, "fp32", 84, cu=cu, raw_k=True)
    inp = _prologue(inp, True, "short4", 84)
    out = _gpu(inp)
    sl = {n: (out[n][:, :61] if n not in ("dS0", "dconv_w") else out[n]) for n in out}
    ins = dict(inp)
    for n in ("q", "k", "v", "g", "beta", "do"):
        ins[n] = inp[n][:, :61]
    _compare(sl, _oracle(ins))


def test_bwd_identity_taps_change_nothing():
    """Taps (0, 0, 0, 1) without SiLU hand every input through unchanged, so every gradient equals that of
    the call without a convolution bit for bit, and dconv_w (the only new output) matches the oracle."""
    _announce("bwd_identity_taps", T=90, H=3, K=64, V=128, seed=85)
    for io in ("fp32", "bf16"):
        inp = _inputs(2, 90, 3, 64, 128, io, 85)
        plain = _gpu(inp)
        w = torch.zeros((3, 2 * 64 + 128, 4), device=DEV)
        w[..., 3] = 1.0
        inp["conv"], inp["conv_w"] = "short4", w
        out = _gpu(inp)
        for n in plain:
            assert torch.equal(out[n], plain[n]), (io, n)
        ref = _oracle(inp)
        assert err(out["dconv_w"], ref["dconv_w"]) <= TOL_FP32


def test_bwd_prologue_empty_batch_zeroes_dconv_w():
    _announce("bwd_prologue_empty", T=0, H=2, K=32, V=32)
    inp = _prologue(_inputs(1, 0, 2, 32, 32, "fp32", 86), True, "short4_silu", 86)
    out = _gpu(inp)
    assert torch.equal(out["dS0"], inp["dS_final"])
    assert torch.equal(out["dconv_w"], torch.zeros_like(out["dconv_w"]))


def test_bwd_prologue_is_deterministic():
    _announce("bwd_prologue_determinism", T=300, H=4, K=128, V=128, seed=87)
    inp = _prologue(_inputs(1, 300, 4, 128, 128, "bf16", 87, raw_k=True), True, "short4_silu", 87)
    a, b = _gpu(inp), _gpu(inp)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_bwd_prologue_4k_workload_sampled_heads():
    # the 4096-token, 96-head bf16 workload with the whole prologue; heads 0 and 95 end to end
    _announce("bwd_prologue_4k", T=4096, H=96, K=128, V=128, io="bf16", seed=1002)
    inp = _inputs(1, 4096, 96, 128, 128, "bf16", 1002, with_S0=False, raw_k=True)
    inp = _prologue(inp, True, "short4_silu", 1002)
    out = _gpu(inp)
    for n in out:
        assert torch.isfinite(out[n]).all(), n
    heads = (0, 95)
    _compare(out, _oracle(inp, heads), heads)
