"""GPU parity of kda_decode_step (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from kda_gated_delta_chunk_amd import chunk_fwd, decode_step
from kda_gated_delta_chunk_amd import synth
from tests.parity import TOL_BF16, TOL_FP32, err, err_stored

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(name, **kw):
    print("\n[case] %s %s" % (name, " ".join("%s=%s" % kv for kv in kw.items())), flush=True)


def _steps(N, H, K, V, io, steps, seed, gate="log_decay", g_scale=1.0, o_gate=False, qk_norm=False):
    S = synth.decode_state(N, H, K, V, seed=seed, device=DEV)
    S_ref = S.double().cpu().numpy()
    worst = {"o": 0.0, "S": 0.0}
    pre = gate == "scaled_sigmoid"
    for step in range(steps):
        inp = synth.decode_inputs(N, H, K, V, io, seed=seed, step=step, device=DEV, gate_preact=pre, g_scale=g_scale,
                                  with_o_gate=o_gate, raw_k=qk_norm)
        args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
        og = inp["o_gate"]
        S32 = S.clone()
        # outputs filled with NaN beforehand: every element must be written
        o = torch.full((N, H, V), float("nan"), dtype=args[0].dtype, device=DEV)
        o32 = torch.full((N, H, V), float("nan"), dtype=torch.float32, device=DEV)
        decode_step(*args, S, out=o, gate=gate, o_gate=og, qk_norm=qk_norm)
        decode_step(*args, S32, o_dtype=torch.float32, out=o32, gate=gate, o_gate=og, qk_norm=qk_norm)
        torch.cuda.synchronize()
        assert torch.equal(S32, S)
        o_ref, S_ref = oracle.decode_step(*(a.cpu() for a in args), S_ref, gate=gate,
                                          o_gate=None if og is None else og.cpu(), qk_norm=qk_norm)
        if io == "fp32":
            worst["o"] = max(worst["o"], err(o.cpu(), o_ref))
        else:
            assert torch.equal(o32.to(torch.bfloat16), o)
            worst["o"] = max(worst["o"], err(o32.cpu(), o_ref), err_stored(o.cpu(), o_ref))
        worst["S"] = max(worst["S"], err(S.cpu(), S_ref))
    print("  errors", worst, flush=True)
    tol = TOL_FP32 if io == "fp32" else TOL_BF16
    assert worst["o"] <= tol and worst["S"] <= tol, worst


@pytest.mark.parametrize("N,H,K,V", [(3, 2, 32, 32), (2, 3, 128, 128), (5, 1, 64, 32), (1, 2, 32, 128),
                                     (2, 2, 128, 64)])
def test_decode_fp32(N, H, K, V):
    _announce("decode_fp32", N=N, H=H, K=K, V=V)
    _steps(N, H, K, V, "fp32", steps=4, seed=31)


@pytest.mark.parametrize("N,H,K,V", [(4, 3, 128, 128), (7, 2, 64, 64)])
def test_decode_bf16(N, H, K, V):
    _announce("decode_bf16", N=N, H=H, K=K, V=V)
    _steps(N, H, K, V, "bf16", steps=4, seed=32)


@pytest.mark.parametrize("io,g_scale", [("fp32", 1.0), ("fp32", 30.0), ("bf16", 1.0), ("bf16", 30.0)])
def test_decode_gate_fused(io, g_scale):
    """g holds the gate pre-activation x (scale 30: most channels saturated at either end); the
    kernel forms -5*sigmoid(x) in fp32, the oracle in fp64."""
    _announce("decode_gate", io=io, g_scale=g_scale)
    _steps(3, 2, 128, 128, io, steps=4, seed=34, gate="scaled_sigmoid", g_scale=g_scale)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_decode_output_gate(io):
    """o * sigmoid(z) with z ~ N(0,1), together with the scaled-sigmoid decay gate."""
    _announce("decode_output_gate", io=io)
    _steps(3, 2, 128, 128, io, steps=4, seed=35, gate="scaled_sigmoid", o_gate=True)


def test_decode_512_streams():
    """N=512, H=96, K=V=128, bf16 inputs, fp32 state (~3.2 GB), 3 consecutive steps, all heads."""
    w = synth.WORKLOADS["decode_512"]
    _announce("decode_512", seed=w.seed)
    _steps(w.N, w.H, w.K, w.V, "bf16", steps=3, seed=w.seed)


@pytest.mark.parametrize("io,N,H,K,V", [("fp32", 1031, 5, 32, 64), ("bf16", 70, 64, 128, 128)])
def test_decode_ragged_pairs_per_workgroup(io, N, H, K, V):
    """More (sequence, head) pairs than one workgroup each (above 4096 pairs a workgroup walks several
    and prefetches the next): N*H not a multiple of the grid, so workgroups take 1 or 2 pairs; both
    gates on, 2 consecutive steps, every pair compared."""
    _announce("decode_ragged_pairs", io=io, N=N, H=H, K=K, V=V)
    _steps(N, H, K, V, io, steps=2, seed=36, gate="scaled_sigmoid", o_gate=True)


@pytest.mark.parametrize("io,N,H,K,V", [("fp32", 3, 2, 128, 128), ("fp32", 5, 3, 32, 64), ("bf16", 4, 3, 128, 128),
                                        ("bf16", 1031, 5, 64, 32)])
def test_decode_qk_norm(io, N, H, K, V):
    """Raw q, k ~ N(0,1) normalised in-kernel, with both gates; the last case walks several pairs per
    workgroup."""
    _announce("decode_qk_norm", io=io, N=N, H=H, K=K, V=V)
    _steps(N, H, K, V, io, steps=3, seed=37, gate="scaled_sigmoid", o_gate=True, qk_norm=True)


def test_decode_steps_equal_prefill():
    """n decode steps from S equal one chunked prefill over the same n tokens from S."""
    _announce("decode_vs_prefill", n=21)
    N, H, K, V, n = 2, 2, 64, 64, 21
    inp = synth.prefill_inputs(N, n, H, K, V, "fp32", seed=33, device=DEV, with_S0=True)
    o_p, S_p = chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S0=inp["S0"])
    S = inp["S0"].clone()
    outs = []
    for t in range(n):
        outs.append(decode_step(*(inp[x][:, t].contiguous() for x in ("q", "k", "v", "g", "beta")), S))
    torch.cuda.synchronize()
    assert err(torch.stack(outs, 1).cpu(), o_p.cpu()) <= TOL_FP32
    assert err(S.cpu(), S_p.cpu()) <= TOL_FP32


# ------------------------------------------------------------ short convolution with a 3-token cache

def _conv_steps(N, H, K, V, io, steps, seed, conv):
    g = torch.Generator().manual_seed(seed)
    w = (0.5 * torch.randn((H, 2 * K + V, 4), generator=g)).to(DEV)
    S = synth.decode_state(N, H, K, V, seed=seed, device=DEV)
    cache = (0.5 * torch.randn((N, H, 3, 2 * K + V), generator=g)).to(synth.DTYPES[io]).to(DEV)
    S_ref = S.double().cpu().numpy()
    c_ref = cache.double().cpu().numpy()
    worst = {"o": 0.0, "S": 0.0}
    for step in range(steps):
        inp = synth.decode_inputs(N, H, K, V, io, seed=seed, step=step, device=DEV, gate_preact=True,
                                  with_o_gate=True, raw_k=True)
        args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
        o = decode_step(*args, S, o_dtype=torch.float32, gate="scaled_sigmoid", o_gate=inp["o_gate"], qk_norm=True,
                        conv=conv, conv_w=w, conv_cache=cache)
        torch.cuda.synchronize()
        o_ref, S_ref, c_ref = oracle.decode_step(*(a.cpu() for a in args), S_ref, gate="scaled_sigmoid",
                                                 o_gate=inp["o_gate"].cpu(), qk_norm=True, conv=conv,
                                                 conv_w=w.cpu(), conv_cache=c_ref)
        # the cache holds raw inputs: it must match exactly
        assert np.array_equal(cache.double().cpu().numpy(), c_ref)
        worst["o"] = max(worst["o"], err(o.cpu(), o_ref))
        worst["S"] = max(worst["S"], err(S.cpu(), S_ref))
    print("  errors", worst, flush=True)
    tol = TOL_FP32 if io == "fp32" else TOL_BF16
    assert worst["o"] <= tol and worst["S"] <= tol, worst


@pytest.mark.parametrize("io,N,H,K,V,conv", [("fp32", 3, 2, 128, 128, "short4"), ("fp32", 5, 3, 32, 64, "short4_silu"),
                                             ("bf16", 4, 3, 128, 128, "short4_silu"),
                                             ("bf16", 1031, 5, 64, 32, "short4")])
def test_decode_conv_cache(io, N, H, K, V, conv):
    """Raw q, k, v convolved over the cached three previous tokens (cache updated in place, compared
    exactly), then normalised, with both gates; the last case walks several pairs per workgroup."""
    _announce("decode_conv", io=io, N=N, H=H, K=K, V=V, conv=conv)
    _conv_steps(N, H, K, V, io, steps=4, seed=38, conv=conv)


def test_prefill_with_conv_hands_over_to_decode():
    """fp32: a convolved prefill over T tokens, then n decode steps whose cache holds the last three raw
    tokens of the prefill, equal one convolved prefill over T + n tokens."""
    _announce("conv_handoff", T=37, n=9)
    N, H, K, V, T, n = 2, 2, 64, 64, 37, 9
    inp = synth.prefill_inputs(N, T + n, H, K, V, "fp32", seed=39, device=DEV, with_S0=True, raw_k=True)
    w = (0.5 * torch.randn((H, 2 * K + V, 4), generator=torch.Generator().manual_seed(39))).to(DEV)
    kw = dict(conv="short4_silu", conv_w=w, qk_norm=True)
    o_all, S_all = chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S0=inp["S0"], **kw)
    head = {x: inp[x][:, :T].contiguous() for x in ("q", "k", "v", "g", "beta")}
    o_p, S = chunk_fwd(head["q"], head["k"], head["v"], head["g"], head["beta"], S0=inp["S0"], **kw)
    cache = torch.cat([inp["q"], inp["k"], inp["v"]], dim=-1)[:, T - 3:T].permute(0, 2, 1, 3).contiguous()
    outs = []
    for t in range(T, T + n):
        outs.append(decode_step(*(inp[x][:, t].contiguous() for x in ("q", "k", "v", "g", "beta")), S,
                                conv_cache=cache, **kw))
    torch.cuda.synchronize()
    assert err(o_p.cpu(), o_all[:, :T].cpu()) <= TOL_FP32
    assert err(torch.stack(outs, 1).cpu(), o_all[:, T:].cpu()) <= TOL_FP32
    assert err(S.cpu(), S_all.cpu()) <= TOL_FP32
