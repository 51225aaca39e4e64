"""Seeded synthetic inputs for the KDA hot path.

This module generates inputs only; it contains none of the method's
arithmetic. It is the single piece shared by the oracle side (tests) and the
product side (benchmark), as both must see identical inputs.

Distributions (the workloads of the spec configurations):
  q, v  ~ N(0, 1)
  k     ~ N(0, 1), then L2-normalised over the key dimension per (token, head)
          in fp32 before the cast to the I/O dtype
  g     = -5 * sigmoid(x), x ~ N(0, 1) per (token, head, key channel): the
          bounded log-retention of the K3 gate (lower bound -5); with
          ``gate_preact=True`` g is the draw x itself (times ``g_scale``), for
          calls that form the log-decay from the pre-activation
  beta  = sigmoid(x), x ~ N(0, 1) per (token, head)
  S0    ~ N(0, 0.02^2) (standard deviation 0.02), fp32
  o_gate ~ N(0, 1) per (token, head, value channel), where asked for: the
          output gate's pre-activation
  do    ~ N(0, 1) per (token, head, value channel): the gradient of a loss
          with respect to o, for the backward pass
  dS_final ~ N(0, 0.02^2), fp32: the gradient with respect to S_final
All draws are fp32 and then rounded to the I/O dtype with round-to-nearest-
even (torch ``.to``). Generation is block-seeded over tokens so a
million-token batch never needs more than one block of fp32 temporaries; a
block's seed is a fixed function of (seed, tensor id, block id).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# tensor ids used in the block seeds
_TID = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "S0": 5, "lengths": 6, "o_gate": 7, "do": 8,
        "dS_final": 9}

DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One named workload of the hot path (sizes as the pages' K3 shapes)."""
    name: str
    kind: str  # "prefill" | "decode"
    H: int
    K: int
    V: int
    io: str
    B: int = 1
    T: int = 0
    chunk: int = 16
    num_seqs: int = 0  # >0: packed varlen batch with this many sequences
    len_lo: int = 0
    len_hi: int = 0
    with_S0: bool = False
    N: int = 0  # decode batch
    steps: int = 0  # decode steps
    seed: int = 0


WORKLOADS = {
    # tiny fp32 prefill the oracle finishes instantly
    "tiny_fp32": Workload("tiny_fp32", "prefill", H=2, K=32, V=32, io="fp32", B=1, T=64, chunk=16, seed=1000),
    # one K3-shaped sequence: 96 heads, 128-dim state channels, 4096 tokens
    "prefill_4k": Workload("prefill_4k", "prefill", H=96, K=128, V=128, io="bf16", B=1, T=4096, chunk=16,
                           seed=1001),
    # 16 packed sequences with lengths uniform in [256, 16384], per-sequence S0
    "varlen_16": Workload("varlen_16", "prefill", H=96, K=128, V=128, io="bf16", num_seqs=16, len_lo=256,
                          len_hi=16384, with_S0=True, chunk=16, seed=1002),
    # 512 concurrent decode streams, one token each, 100 steps
    "decode_512": Workload("decode_512", "decode", H=96, K=128, V=128, io="bf16", N=512, steps=100, seed=1003),
    # one million-token sequence
    "prefill_1m": Workload("prefill_1m", "prefill", H=96, K=128, V=128, io="bf16", B=1, T=1 << 20, chunk=16,
                           seed=1004),
}


def block_seed(seed: int, tensor: str, block: int) -> int:
    """Deterministic 63-bit seed for one block of one tensor."""
    ss = np.random.SeedSequence([int(seed), _TID[tensor], int(block)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _randn(shape, seed: int, tensor: str, block: int, device) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(block_seed(seed, tensor, block))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def varlen_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> list[int]:
    """Sequence lengths uniform on [lo, hi] (inclusive), device independent."""
    rng = np.random.default_rng([int(seed), _TID["lengths"], 0])
    return [int(x) for x in rng.integers(lo, hi, size=num_seqs, endpoint=True)]


def cu_from_lengths(lengths) -> list[int]:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu


def prefill_inputs(B: int, T: int, H: int, K: int, V: int, io: str = "bf16", seed: int = 0,
                   device="cpu", cu_seqlens=None, with_S0: bool = False, block_tokens: int = 65536,
                   g_shift: float = 0.0, g_const: float | None = None, beta_const: float | None = None,
                   gate_preact: bool = False, g_scale: float = 1.0, with_o_gate: bool = False,
                   raw_k: bool = False):
    """Inputs of one prefill call.

    Returns a dict with q, k, g [B,T,H,K], v [B,T,H,V], beta [B,T,H] in the I/O
    dtype, S0 [N,H,K,V] fp32 (or None) and cu_seqlens int32 [N+1] (or None).
    ``g_shift`` moves the pre-sigmoid draw of g (e.g. -6 for mild decay);
    ``g_const``/``beta_const`` replace the draw by a constant (stress cases);
    ``gate_preact`` stores the pre-sigmoid draw g_scale * x + g_shift itself;
    ``with_o_gate`` adds an output-gate pre-activation ``o_gate`` [B,T,H,V];
    ``raw_k`` keeps the N(0, 1) draw of k as it is (no normalisation; for
    calls that normalise q and k themselves).
    """
    dt = DTYPES[io]
    dev = torch.device(device)
    q = torch.empty((B, T, H, K), dtype=dt, device=dev)
    k = torch.empty_like(q)
    g = torch.empty_like(q)
    v = torch.empty((B, T, H, V), dtype=dt, device=dev)
    beta = torch.empty((B, T, H), dtype=dt, device=dev)
    og = torch.empty((B, T, H, V), dtype=dt, device=dev) if with_o_gate else None
    flat = B * T
    qf, kf, gf = q.view(flat, H, K), k.view(flat, H, K), g.view(flat, H, K)
    vf, bf = v.view(flat, H, V), beta.view(flat, H)
    nblk = (flat + block_tokens - 1) // block_tokens
    for blk in range(nblk):
        a, b = blk * block_tokens, min(flat, (blk + 1) * block_tokens)
        n = b - a
        qf[a:b] = _randn((n, H, K), seed, "q", blk, dev).to(dt)
        kr = _randn((n, H, K), seed, "k", blk, dev)
        if not raw_k:
            kr = kr / torch.sqrt(torch.sum(kr * kr, dim=-1, keepdim=True))
        kf[a:b] = kr.to(dt)
        del kr
        vf[a:b] = _randn((n, H, V), seed, "v", blk, dev).to(dt)
        if og is not None:
            og.view(flat, H, V)[a:b] = _randn((n, H, V), seed, "o_gate", blk, dev).to(dt)
        if g_const is not None:
            gf[a:b] = torch.full((n, H, K), float(g_const), device=dev).to(dt)
        elif gate_preact:
            gf[a:b] = (g_scale * _randn((n, H, K), seed, "g", blk, dev) + g_shift).to(dt)
        else:
            gf[a:b] = (-5.0 * torch.sigmoid(_randn((n, H, K), seed, "g", blk, dev) + g_shift)).to(dt)
        if beta_const is not None:
            bf[a:b] = torch.full((n, H), float(beta_const), device=dev).to(dt)
        else:
            bf[a:b] = torch.sigmoid(_randn((n, H), seed, "beta", blk, dev)).to(dt)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = torch.as_tensor(list(cu_seqlens), dtype=torch.int32, device=dev)
        N = cu.numel() - 1
    S0 = None
    if with_S0:
        S0 = 0.02 * _randn((N, H, K, V), seed, "S0", 0, dev)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "S0": S0, "cu_seqlens": cu, "o_gate": og}


def output_grads(B: int, T: int, H: int, V: int, io: str = "bf16", seed: int = 0, device="cpu",
                 num_seqs: int = 0, K: int = 0, block_tokens: int = 65536):
    """Gradients fed to a backward call: do [B,T,H,V] in the I/O dtype and, when
    num_seqs and K are given, dS_final [num_seqs,H,K,V] fp32 (else None)."""
    dt = DTYPES[io]
    dev = torch.device(device)
    do = torch.empty((B, T, H, V), dtype=dt, device=dev)
    flat = B * T
    df = do.view(flat, H, V)
    for blk in range((flat + block_tokens - 1) // block_tokens):
        a, b = blk * block_tokens, min(flat, (blk + 1) * block_tokens)
        df[a:b] = _randn((b - a, H, V), seed, "do", blk, dev).to(dt)
    dsf = None
    if num_seqs and K:
        dsf = 0.02 * _randn((num_seqs, H, K, V), seed, "dS_final", 0, dev)
    return do, dsf


def workload_prefill_inputs(w: Workload, device="cpu", **kw):
    """Inputs of a named prefill workload."""
    if w.num_seqs:
        lengths = varlen_lengths(w.num_seqs, w.len_lo, w.len_hi, w.seed)
        cu = cu_from_lengths(lengths)
        return prefill_inputs(1, cu[-1], w.H, w.K, w.V, w.io, w.seed, device, cu_seqlens=cu,
                              with_S0=w.with_S0, **kw)
    return prefill_inputs(w.B, w.T, w.H, w.K, w.V, w.io, w.seed, device, with_S0=w.with_S0, **kw)


def decode_inputs(N: int, H: int, K: int, V: int, io: str = "bf16", seed: int = 0, step: int = 0,
                  device="cpu", gate_preact: bool = False, g_scale: float = 1.0, with_o_gate: bool = False,
                  raw_k: bool = False):
    """Per-step decode inputs q, k, g [N,H,K], v [N,H,V], beta [N,H] (step = block id).
    ``gate_preact``: g is the pre-sigmoid draw g_scale * x itself; ``with_o_gate``: also an
    output-gate pre-activation o_gate [N,H,V] (else None); ``raw_k``: k is the N(0, 1) draw
    itself, not normalised."""
    dt = DTYPES[io]
    dev = torch.device(device)
    q = _randn((N, H, K), seed, "q", step, dev).to(dt)
    kr = _randn((N, H, K), seed, "k", step, dev)
    k = (kr if raw_k else kr / torch.sqrt(torch.sum(kr * kr, dim=-1, keepdim=True))).to(dt)
    v = _randn((N, H, V), seed, "v", step, dev).to(dt)
    x = _randn((N, H, K), seed, "g", step, dev)
    g = (g_scale * x if gate_preact else -5.0 * torch.sigmoid(x)).to(dt)
    beta = torch.sigmoid(_randn((N, H), seed, "beta", step, dev)).to(dt)
    og = _randn((N, H, V), seed, "o_gate", step, dev).to(dt) if with_o_gate else None
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "o_gate": og}


def decode_state(N: int, H: int, K: int, V: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Initial decode state [N,H,K,V] fp32, entries N(0, 0.02^2)."""
    return 0.02 * _randn((N, H, K, V), seed, "S0", 0, torch.device(device))
