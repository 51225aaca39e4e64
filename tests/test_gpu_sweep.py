"""A seeded sweep over combinations of the prefill's and the backward's options on the GPU, against the fp64
oracle: I/O dtype, head sizes, batched or packed sequences (empty and one-token ones included), chunk size,
both gates, the q/k normalisation, the short convolution (with and without SiLU), an initial state, the operand
format and the fused low-memory form. Each case is drawn from its own seed, so a failing case reruns alone.
The targeted tests cover each option's edge cases; this sweep covers their interactions.
"""
import numpy as np
import pytest
import torch

from kda_gated_delta_chunk_amd import synth
from tests import test_gpu_backward as bwd
from tests.test_gpu_prefill import _announce, _check, _run_low_memory

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 24


def _case(i):
    rng = np.random.default_rng(7000 + i)
    c = {"io": ["fp32", "bf16"][rng.integers(2)], "K": int(rng.choice([32, 64, 128])),
         "V": int(rng.choice([32, 64, 128])), "H": int(rng.integers(1, 4)), "chunk": int(rng.choice([16, 64])),
         "gate": ["log_decay", "scaled_sigmoid"][rng.integers(2)], "o_gate": bool(rng.integers(2)),
         "qk_norm": bool(rng.integers(2)), "conv": ["none", "short4", "short4_silu"][rng.integers(3)],
         "S0": bool(rng.integers(2)), "seed": 7000 + i}
    if rng.integers(2):  # packed: some empty and one-token sequences
        lengths = [int(x) for x in rng.integers(0, 180, size=int(rng.integers(1, 6)))]
        for j in range(len(lengths)):
            if rng.random() < 0.2:
                lengths[j] = int(rng.choice([0, 1, 2]))
        c["lengths"] = lengths
    else:
        c["B"], c["T"] = int(rng.integers(1, 4)), int(rng.integers(1, 260))
    plain16 = c["io"] == "bf16" and c["chunk"] == 16 and c["conv"] == "none"
    c["operands"] = "fp16" if plain16 and rng.random() < 0.3 else "bf16"
    c["low_memory"] = c["chunk"] == 16 and c["conv"] == "none" and rng.random() < 0.3
    return c


def _inputs(c):
    if "lengths" in c:
        cu = synth.cu_from_lengths(c["lengths"])
        B, T = 1, cu[-1]
    else:
        cu, B, T = None, c["B"], c["T"]
    inp = synth.prefill_inputs(B, T, c["H"], c["K"], c["V"], c["io"], seed=c["seed"], device=DEV, cu_seqlens=cu,
                               with_S0=c["S0"], gate_preact=c["gate"] == "scaled_sigmoid",
                               with_o_gate=c["o_gate"], raw_k=c["qk_norm"])
    inp["gate"] = c["gate"]
    inp["qk_norm"] = c["qk_norm"]
    if c["conv"] != "none":
        g = torch.Generator().manual_seed(c["seed"])
        inp["conv"] = c["conv"]
        inp["conv_w"] = (0.5 * torch.randn((c["H"], 2 * c["K"] + c["V"], 4), generator=g)).to(DEV)
    inp["operands"] = c["operands"]
    return inp


@pytest.mark.parametrize("i", range(N_CASES))
def test_prefill_option_sweep(i):
    c = _case(i)
    _announce("sweep_prefill", **c)
    inp = _inputs(c)
    o, Sf = _check(inp, io=c["io"], chunk=c["chunk"])
    if c["low_memory"]:  # the fused form with the least workspace gives the two-pass result bit for bit
        o2, S2 = _run_low_memory(inp, operands=c["operands"])
        assert torch.equal(o, o2) and torch.equal(Sf, S2)


@pytest.mark.parametrize("i", range(N_CASES))
def test_backward_option_sweep(i):
    c = _case(i)
    _announce("sweep_backward", **c)
    inp = _inputs(c)
    B, T = inp["q"].shape[:2]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    inp["do"], inp["dS_final"] = synth.output_grads(B, T, c["H"], c["V"], c["io"], c["seed"], DEV, num_seqs=N,
                                                    K=c["K"])
    out = bwd._gpu(inp)
    assert ("dconv_w" in out) == (c["conv"] != "none") and ("do_gate" in out) == c["o_gate"]
    bwd._compare(out, bwd._oracle(inp))
