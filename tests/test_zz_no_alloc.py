"""kda_chunk_fwd_no_alloc (the prefill without a workspace argument, for callers that cannot allocate)
against kda_chunk_fwd through the C ABI: two calls in a row on the library's device scratch, the second
smaller, each equal bit for bit to kda_chunk_fwd with a workspace of the scratch's size (the same path:
fused when the two passes do not fit, two passes when they do), on outputs filled with NaN beforehand.
"""
import ctypes

import pytest
import torch

from kda_gated_delta_chunk_amd import _lib, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
IO = {"fp32": 0, "bf16": 1}


def _announce(name, **kw):
    print("\n[case] %s %s" % (name, " ".join("%s=%s" % kv for kv in kw.items())), flush=True)


def _p(t):
    return None if t is None else t.data_ptr()


def _call(inp, io, o, Sf, ws=None, gate=0):
    lib = _lib.load()
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    cu = inp["cu_seqlens"]
    N = B if cu is None else cu.numel() - 1
    head = [_p(inp[n]) for n in ("q", "k", "v", "g", "beta", "o_gate")] + [_p(inp["S0"]), _p(cu), B, T, H, K, V, N,
                                                                              16, IO[io], gate, 0, 0, None, 0, IO[io],
                                                                              o.data_ptr(), Sf.data_ptr()]
    stream = torch.cuda.current_stream(DEV).cuda_stream
    if ws is None:
        st = lib.kda_chunk_fwd_no_alloc(*head, stream)
        what = "kda_chunk_fwd_no_alloc"
    else:
        st = lib.kda_chunk_fwd(*head, ws.data_ptr(), ws.numel(), stream)
        what = "kda_chunk_fwd"
    _lib.check(st, what)
    torch.cuda.synchronize()


def _nan_like(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _both(inp, io, gate=0):
    """(o, S_final) of the no-alloc call and of kda_chunk_fwd with a workspace of the scratch's size."""
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    dt = inp["q"].dtype
    o1, S1 = _nan_like((B, T, H, V), dt), _nan_like((N, H, K, V), torch.float32)
    _call(inp, io, o1, S1, gate=gate)
    ws = torch.full((_lib.NO_ALLOC_SCRATCH_BYTES,), 0xFF, dtype=torch.uint8, device=DEV)
    o2, S2 = _nan_like((B, T, H, V), dt), _nan_like((N, H, K, V), torch.float32)
    _call(inp, io, o2, S2, ws=ws, gate=gate)
    return (o1, S1), (o2, S2)


def _two_pass_fits(B, T, H, K, V, N, io):
    lib = _lib.load()
    need = lib.kda_chunk_fwd_workspace_bytes(B, T, H, K, V, N, 16, IO[io], 0, 0)
    return need <= _lib.NO_ALLOC_SCRATCH_BYTES


def test_no_alloc_matches_kda_chunk_fwd_on_two_calls_in_a_row():
    # first call: 4096 tokens x 16 heads, too large for the two passes in the scratch -> the fused kernel
    _announce("no_alloc_large", T=4096, H=16, K=128, V=128, io="bf16", seed=91)
    big = synth.prefill_inputs(1, 4096, 16, 128, 128, "bf16", seed=91, device=DEV, with_S0=True)
    assert not _two_pass_fits(1, 4096, 16, 128, 128, 1, "bf16")
    (o1, S1), (o2, S2) = _both(big, "bf16")
    assert not torch.isnan(o1).any() and not torch.isnan(S1).any()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    del big
    # second call, smaller: packed sequences (an empty one), both gates -> the two passes fit in the scratch
    cu = [0, 5, 5, 200, 333]
    _announce("no_alloc_small", cu=cu, H=4, K=128, V=64, io="bf16", seed=92)
    small = synth.prefill_inputs(1, cu[-1], 4, 128, 64, "bf16", seed=92, device=DEV, cu_seqlens=cu,
                                 with_S0=True, gate_preact=True, with_o_gate=True)
    assert _two_pass_fits(1, cu[-1], 4, 128, 64, len(cu) - 1, "bf16")
    (o1, S1), (o2, S2) = _both(small, "bf16", gate=1)
    assert not torch.isnan(o1).any() and not torch.isnan(S1).any()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_no_alloc_fp32_ragged_batch():
    _announce("no_alloc_fp32", B=3, T=77, H=2, K=64, V=32, io="fp32", seed=93)
    inp = synth.prefill_inputs(3, 77, 2, 64, 32, "fp32", seed=93, device=DEV, with_S0=True)
    (o1, S1), (o2, S2) = _both(inp, "fp32")
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_no_alloc_refuses_a_call_whose_least_workspace_exceeds_the_scratch():
    # a convolution keeps the convolved q, k and v in the workspace: 4096 x 8 heads need ~50 MB
    lib = _lib.load()
    B, T, H, K, V = 1, 4096, 8, 128, 128
    assert lib.kda_chunk_fwd_min_workspace_bytes(B, T, H, K, V, 1, 16, 1, 2, 0) > _lib.NO_ALLOC_SCRATCH_BYTES
    x = torch.zeros(16, device=DEV)
    st = lib.kda_chunk_fwd_no_alloc(_p(x), _p(x), _p(x), _p(x), _p(x), None, None, None, B, T, H, K, V, 1, 16, 1, 0,
                                    0, 2, _p(x), 0, 1, _p(x), _p(x), None)
    assert st == 3  # KDA_ERROR_WORKSPACE_TOO_SMALL, before any launch
