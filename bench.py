"""Benchmark of the MI355X KDA hot path on one GPU; prints ONE JSON line.

A step is one kda_chunk_fwd call on the K3-shaped workload: B=1, T=4096, H=96,
K=V=128, bf16 q/k/v/g/beta, chunk 16, zero initial state, default (bf16)
state-pass operands, returning o and S_final. Inputs are seeded synthetic
tensors already resident in HBM. Before anything is timed the headline step
runs back to back for --settle-s seconds (the GPU clock needs tens of
milliseconds of load to settle). `value` is prefill tokens/s. Further legs:
chunk 64, fp16 operands, the gate/norm/convolution prologues and the output
gate, the 16-sequence packed workload (about 130K tokens) and the
1,048,576-token sequence. The decode half of the metric (N=512 streams, H=96,
fp32 state of ~3.2 GB updated in place, 100 consecutive steps) is reported
under "decode". The backward pass (kda_chunk_bwd) on the prefill workload's
inputs is reported under "backward", against the fp32 dense matrix-core peak
(its products run as fp32 MFMA).

Kernel durations come from HIP events recorded on the stream the kernels run
on, around each phase of every timed step. Roofline figures use algorithmic
bytes (the tensors the operation must read and write once) divided by those
durations, against MI355X's published 8 TB/s HBM3E bandwidth.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import torch

from kda_gated_delta_chunk_amd import _lib, decode_step, synth, workspace_status
from kda_gated_delta_chunk_amd.source_hash import csrc_hash

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix, TFLOP/s
FP32_MFMA_PEAK_TFS = 157.3      # MI355X dense fp32 matrix cores, TFLOP/s
SIMDS = 256 * 4                 # MI355X: 256 compute units of 4 SIMDs (one matrix core each)
CLOCK_HZ = 2.4e9                # peak engine clock


def prefill_algorithmic_bytes(T, H, K, V, N, es=2, with_S0=False):
    """Bytes the prefill must move once: q, k, g, v, beta in, o out, S_final out (S0 in)."""
    per_tok = H * (3 * K * es + V * es + es + V * es)
    states = N * H * K * V * 4 * (2 if with_S0 else 1)
    return T * per_tok + states, {"prep": T * H * (3 * K * es + es),
                                  "state": T * H * 2 * V * es + states}


def prefill_flops(T, H, K, V, C=16):
    """Algorithmic flops of the chunk form per token-head: 6dK (W, state update, Q*S) plus the
    intra-chunk products and the solve (triangles counted as triangles)."""
    d = K
    per = 6 * d * V + (5 * C + 3) * d + d * d / C + C * C / 3
    return T * H * per


class PrefillLeg:
    """One prefill workload on the GPU: inputs resident in HBM, preallocated outputs and workspaces, and
    the three ABI calls (kda_chunk_fwd, and the split kda_chunk_prep / kda_chunk_state) as closures."""

    def __init__(self, dev, inp, chunk=16, gate="log_decay", qk_norm=False, conv="none", operands="bf16",
                 with_split=True, low_memory=False):
        lib = self.lib = _lib.load()
        self.inp = inp
        gc = _lib.GATES[gate]
        qkc = _lib.KDA_QK_L2NORM if qk_norm else _lib.KDA_QK_AS_GIVEN
        og = inp["o_gate"].data_ptr() if inp.get("o_gate") is not None else None
        B, T, H, K = inp["q"].shape
        V = inp["v"].shape[-1]
        cu = inp.get("cu_seqlens")
        N = B if cu is None else cu.numel() - 1
        self.B, self.T, self.H, self.K, self.V, self.N = B, T, H, K, V, N
        cup = None if cu is None else cu.data_ptr()
        s0 = None if inp.get("S0") is None else inp["S0"].data_ptr()
        io = 1 if inp["q"].dtype == torch.bfloat16 else 0  # kda_dtype_t of the inputs (and of o)
        self.o = torch.empty((B, T, H, V), dtype=inp["q"].dtype, device=dev)
        self.Sf = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
        cc = _lib.CONVS[conv]
        oc = _lib.OPERANDS[operands]
        cw = None
        if conv != "none":
            cw = (0.5 * torch.randn((H, 2 * K + V, 4), generator=torch.Generator().manual_seed(7))).to(dev)
        cwp = None if cw is None else cw.data_ptr()
        self.cw = cw
        query = lib.kda_chunk_fwd_min_workspace_bytes if low_memory else lib.kda_chunk_fwd_workspace_bytes
        self.wsb = query(B, T, H, K, V, N, chunk, io, cc, oc)
        self.ws = torch.empty(self.wsb, dtype=torch.uint8, device=dev)
        self.swsb = lib.kda_chunk_prep_workspace_bytes(B, T, H, K, V, N, chunk, io, cc, oc) if with_split else 0
        self.sws = torch.empty(self.swsb, dtype=torch.uint8, device=dev) if with_split else None
        self.stream = torch.cuda.current_stream(dev)
        sh = self.stream.cuda_stream
        p = {n: inp[n].data_ptr() for n in ("q", "k", "v", "g", "beta")}
        o, Sf = self.o.data_ptr(), self.Sf.data_ptr()

        def fwd():
            _lib.check(lib.kda_chunk_fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], og, s0, cup, B, T, H, K, V, N,
                                         chunk, io, gc, qkc, cc, cwp, oc, io, o, Sf, self.ws.data_ptr(), self.wsb, sh),
                       "kda_chunk_fwd")

        def prep():
            _lib.check(lib.kda_chunk_prep(p["q"], p["k"], p["g"], p["beta"], cup, B, T, H, K, V, N, chunk, io, gc, qkc,
                                          cc, cwp, oc, self.sws.data_ptr(), self.swsb, sh), "kda_chunk_prep")

        def state():
            _lib.check(lib.kda_chunk_state(p["v"], og, s0, cup, B, T, H, K, V, N, chunk, io, cc, cwp, io, o, Sf,
                                           self.sws.data_ptr(), self.swsb, sh), "kda_chunk_state")

        self.fwd, self.prep, self.state = fwd, prep, state

    def device_error(self):
        """Error bits the kernels recorded in the workspaces (0: none)."""
        e = workspace_status(self.ws)
        if self.sws is not None:
            e |= workspace_status(self.sws)
        return e

    def time_fwd(self, steps, warmup):
        """The step: one kda_chunk_fwd call. Returns (wall ms per step, event ms per step)."""
        for _ in range(warmup):
            self.fwd()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(self.stream)
        for _ in range(steps):
            self.fwd()
        ev[1].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / steps, ev[0].elapsed_time(ev[1]) / steps

    def time_split(self, steps, warmup):
        """Per-kernel durations: the two halves as separate calls, HIP events on the launch stream around
        each. Returns (prep ms, state ms) averaged over the steps."""
        for _ in range(warmup):
            self.prep()
            self.state()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev[i][0].record(self.stream)
            self.prep()
            ev[i][1].record(self.stream)
            self.state()
            ev[i][2].record(self.stream)
        torch.cuda.synchronize()
        return (sum(e[0].elapsed_time(e[1]) for e in ev) / steps,
                sum(e[1].elapsed_time(e[2]) for e in ev) / steps)


def settle_clock(leg, seconds):
    """Runs the headline step back to back for `seconds` of wall time before anything is timed: the GPU's
    clock needs some tens of milliseconds of load to reach its steady state, and the first timed leg
    would otherwise run on a rising clock."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(20):
            leg.fwd()
        n += 20
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return {"seconds": time.perf_counter() - t0, "calls": n}


def time_decode(w, steps, dev, gate="log_decay", qk_norm=False):
    N, H, K, V = w.N, w.H, w.K, w.V
    S = synth.decode_state(N, H, K, V, seed=w.seed, device=dev)
    inputs = [synth.decode_inputs(N, H, K, V, w.io, seed=w.seed, step=s, device=dev,
                                  gate_preact=(gate == "scaled_sigmoid"), raw_k=qk_norm) for s in range(steps)]
    o = torch.empty((N, H, V), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    for s in range(2):  # warm-up on the same state (its values only drift)
        decode_step(*(inputs[s][n] for n in ("q", "k", "v", "g", "beta")), S, out=o, gate=gate, qk_norm=qk_norm)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for s in range(steps):
        decode_step(*(inputs[s][n] for n in ("q", "k", "v", "g", "beta")), S, out=o, gate=gate, qk_norm=qk_norm)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[s].elapsed_time(ev[s + 1]) for s in range(steps))
    total = ev[0].elapsed_time(ev[steps])
    bytes_step = N * H * (2 * K * V * 4 + (3 * K + V + 1) * 2 + V * 2)
    return {"steps": steps, "total_ms": total, "ms_per_step": total / steps, "median_ms": per[len(per) // 2],
            "bytes_per_step": bytes_step, "N": N, "H": H}


def time_copy(dev, nbytes=2 << 30, reps=10):
    """A plain device-to-device copy of nbytes (torch's copy kernel): the HBM rate a streaming kernel
    reaches on this GPU (bytes read + bytes written per second), as a reference for the rooflines."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(reps):
        dst.copy_(src)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes_copied": nbytes, "ms": ms, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def backward_flops(T, H, K, V):
    """Algorithmic flops of the backward per call, counted on the per-token reverse recurrence: one forward
    recompute (decay, read, write: 5KV) plus the reverse step (G += q do^T, S_t do, G^T k, beta G d - A dv,
    G - k dv^T, rowsum(GA * A), decay: 19KV). The chunk form the library runs performs about 16KV per token
    plus O(16 (K + V)), some 0.78 of this count at K = V = 128."""
    return 24 * K * V * T * H


def time_backward(w, steps, warmup, dev, prologue=False, segment_tokens=0, o_gate=False):
    """kda_chunk_bwd on the prefill workload's inputs, dL/do ~ N(0, 1), no dL/dS_final. prologue: the
    forward normalised q and k and ran the short convolution with SiLU (raw k, taps ~ N(0, 0.5^2)), so the
    gradients also run back through both and dL/d(taps) is formed. segment_tokens: a workspace of the size
    for segments of that many tokens, so the call runs in segments. o_gate: the forward gated its output,
    o = core * sigmoid(z) with z ~ N(0, 1), so dL/dz is formed too."""
    lib = _lib.load()
    inp = synth.workload_prefill_inputs(w, device=dev, raw_k=prologue)
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    do, _ = synth.output_grads(B, T, H, V, w.io, w.seed, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty((B, T, H, K), **f32) for _ in range(3)] + [torch.empty((B, T, H, V), **f32),
                                                                    torch.empty((B, T, H), **f32)]
    dq, dk, dg, dv, db = (t.data_ptr() for t in outs)
    dS0 = torch.empty((B, H, K, V), **f32)
    z = torch.randn((B, T, H, V), generator=torch.Generator().manual_seed(11)).to(dev, inp["v"].dtype) if o_gate else None
    dz = torch.empty((B, T, H, V), **f32) if o_gate else None
    zp, dzp = (z.data_ptr(), dz.data_ptr()) if o_gate else (None, None)
    qc, cc = (_lib.KDA_QK_L2NORM, _lib.CONVS["short4_silu"]) if prologue else (0, 0)
    cw = (0.5 * torch.randn((H, 2 * K + V, 4), generator=torch.Generator().manual_seed(7))).to(dev) if prologue else None
    dcw = torch.empty((H, 2 * K + V, 4), **f32) if prologue else None
    cwp, dcwp = (cw.data_ptr(), dcw.data_ptr()) if prologue else (None, None)
    if segment_tokens:
        wsb = lib.kda_chunk_bwd_segmented_workspace_bytes(B, T, H, K, V, B, qc, cc, segment_tokens)
    else:
        wsb = lib.kda_chunk_bwd_workspace_bytes(B, T, H, K, V, B, qc, cc)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p = {n: inp[n].data_ptr() for n in ("q", "k", "v", "g", "beta")}

    def bwd():
        _lib.check(lib.kda_chunk_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], zp, None, None, do.data_ptr(),
                                     None, B, T, H, K, V, B, 1, 0, qc, cc, cwp, dq, dk, dv, dg, db, dzp, dcwp,
                                     dS0.data_ptr(), ws.data_ptr(), wsb, stream.cuda_stream), "kda_chunk_bwd")

    for _ in range(warmup):
        bwd()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        bwd()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[steps]) / steps
    return {"B": B, "T": T, "H": H, "K": K, "V": V, "ms": ms, "ws_bytes": wsb}


def measured_counter(kernel_prefix, field="traffic_bytes"):
    """A per-launch counter figure of a kernel from the committed counter summary
    (profiles/traffic.json): HBM bytes ("traffic_bytes") or matrix-core busy cycles summed over
    the device ("mfma_busy_cycles"); None if the kernels changed since it was taken."""
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("csrc_hash") != csrc_hash():
        return None
    for name, v in t["kernels"].items():
        if name.startswith(kernel_prefix):
            return v.get(field)
    return None


def measured_traffic(kernel_prefix):
    return measured_counter(kernel_prefix, "traffic_bytes")


def mfma_busy_frac(kernel_prefix, ms):
    """Matrix-core busy fraction of the whole chip over a launch of `ms` milliseconds, from the
    rocprof SQ_VALU_MFMA_BUSY_CYCLES per launch in profiles/traffic.json (None if absent or stale)."""
    cyc = measured_counter(kernel_prefix, "mfma_busy_cycles")
    if cyc is None or not ms:
        return None
    return cyc / (ms * 1e-3 * CLOCK_HZ * SIMDS)


def mfma_from_counters(sq_csv, out_path):
    """Add each kda kernel's SQ_VALU_MFMA_BUSY_CYCLES per launch (summed over the device; average over its
    first bench leg, as the byte counters) from a rocprofv3 counter run of `bench.py --counters` to the
    counter summary, if that summary was taken on the same kernel sources."""
    import csv
    from collections import defaultdict
    with open(out_path) as fh:
        out = json.load(fh)
    if out.get("csrc_hash") != csrc_hash():
        raise SystemExit("%s was taken on other kernel sources; take FETCH_SIZE/WRITE_SIZE again first" % out_path)
    vals = defaultdict(list)
    rows = sorted(csv.DictReader(open(sq_csv)), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        if "kda" in name and r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
            vals[name].append(float(r["Counter_Value"]))
    for k, v in vals.items():
        out["kernels"].setdefault(k, {})["mfma_busy_cycles"] = sum(v[:3]) / len(v[:3])
    with open(out_path, "w") as fh:
        fh.write(json.dumps(out, indent=1) + "\n")
    return out


def traffic_from_counters(fetch_csv, write_csv, out_path):
    """Per-launch HBM bytes of each kda kernel from two rocprofv3 counter runs of
    `bench.py --counters` (FETCH_SIZE, then WRITE_SIZE; values in KiB per dispatch), each
    scaled by what the same counter reads for the run's 1 GiB device copy; written as JSON
    together with the hash of the kernel sources it was measured on."""
    import csv
    from collections import defaultdict
    copy_bytes = 1 << 30

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration copy is the run's first device copy of at least 256 MiB
        copy = next(float(r["Counter_Value"]) for r in rows
                    if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) * 1024.0 >= (1 << 28))
        vals = defaultdict(list)
        for r in rows:
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            if "kda" in name:
                vals[name].append(float(r["Counter_Value"]))
        # per kernel: its first bench leg (the first three dispatches: one warm-up and two steps of the first
        # leg that runs it; for the chunk-16 kernels that leg is the headline) and the average over all legs
        return copy, {k: (sum(v[:3]) / len(v[:3]), sum(v) / len(v)) for k, v in vals.items()}

    fcopy, f = per_kernel(fetch_csv, "FETCH_SIZE")
    wcopy, w = per_kernel(write_csv, "WRITE_SIZE")
    fscale = copy_bytes / (fcopy * 1024.0)  # the copy reads and writes 1 GiB
    wscale = copy_bytes / (wcopy * 1024.0)
    out = {"csrc_hash": csrc_hash(), "fetch_scale": fscale, "write_scale": wscale, "kernels": {}}
    for k in sorted(set(f) | set(w)):
        fb, fa = (x * 1024.0 * fscale for x in f.get(k, (0.0, 0.0)))
        wb, wa = (x * 1024.0 * wscale for x in w.get(k, (0.0, 0.0)))
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
                             "traffic_bytes_all_legs": fa + wa}
    with open(out_path, "w") as fh:
        fh.write(json.dumps(out, indent=1) + "\n")
    return out


def cpu_baseline(w):
    """The fp64 oracle on the host, on the full 4096-token, 96-head prefill workload (generation excluded),
    on every host core it may use, and on one core over a two-head sample of the same workload (scaled to
    tokens of all heads)."""
    import oracle  # test infrastructure: only this baseline leg uses it
    inp = synth.workload_prefill_inputs(w, device="cpu")
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    oracle.chunk_fwd(*args, threads=threads)
    dt = time.perf_counter() - t0
    B, T, H, _ = args[0].shape
    hs = [0, H - 1]
    sample = [a[:, :, hs].contiguous() for a in args]
    t0 = time.perf_counter()
    oracle.chunk_fwd(*sample, threads=1)
    dt1 = time.perf_counter() - t0
    return {"value": B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "full workload: B=1 T=%d H=%d K=V=128 bf16 inputs, fp64 per-token recurrence, %.2f s wall "
                      "on %d threads" % (T, H, dt, threads),
            "one_core": {"value": B * T * len(hs) / H / dt1, "unit": "tokens/s (of all %d heads)" % H, "cores": 1,
                         "sample": "heads %s of the same workload, %.2f s on one thread" % (hs, dt1)}}


def leg_summary(leg, wall_ms, ev_ms, name, C=16, split=None):
    """Throughput and whole-path roofline of one timed leg."""
    T = leg.B * leg.T
    has_S0 = leg.inp.get("S0") is not None
    path_bytes, kb = prefill_algorithmic_bytes(T, leg.H, leg.K, leg.V, leg.N, es=leg.o.element_size(), with_S0=has_S0)
    gbs = path_bytes / (ev_ms * 1e-3) / 1e9
    tf = prefill_flops(T, leg.H, leg.K, leg.V, C) / (ev_ms * 1e-3) / 1e12
    out = {"workload": name, "tokens_per_s": T / (wall_ms * 1e-3), "ms_per_step": wall_ms, "event_ms": ev_ms,
           "roofline_path": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": path_bytes,
                             "mfma_tflops_algorithmic": tf, "mfma_frac_algorithmic": tf / BF16_PEAK_TFLOPS},
           "workspace_bytes": leg.wsb}
    if split is not None:
        out["split_calls_ms"] = {"kda_chunk_prep": split[0], "kda_chunk_state": split[1]}
    return out, kb


def run_config(idx, args, dev, say):
    """One workload of the five preset configurations, timed as in the full run."""
    names = {0: "tiny_fp32", 1: "prefill_4k", 2: "varlen_16", 3: "decode_512", 4: "prefill_1m"}
    w = synth.WORKLOADS[names[idx]]
    out = {"config_index": idx, "workload": w.name, "steps": args.steps, "warmup": args.warmup}
    if w.kind == "decode":
        say("decode %s: %d steps" % (w.name, args.decode_steps))
        d = time_decode(w, args.decode_steps, dev)
        gbs = d["bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9
        out.update({"ms_per_step": d["ms_per_step"], "tokens_per_s": d["N"] / (d["ms_per_step"] * 1e-3),
                    "GB_per_s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS})
        return out
    inp = synth.workload_prefill_inputs(w, device=dev)
    large = w.B * w.T * w.H > (1 << 26)
    low_memory = False
    if large:  # the two passes only when their workspace fits beside the inputs
        free, _ = torch.cuda.mem_get_info()
        wsb = _lib.load().kda_chunk_fwd_workspace_bytes(w.B, w.T, w.H, w.K, w.V, 1, 16, 1, 0, 0)
        low_memory = wsb + (4 << 30) > free
    leg = PrefillLeg(dev, inp, with_split=not large, low_memory=low_memory)
    if args.settle_s > 0 and not large:
        out["clock_settle"] = settle_clock(leg, args.settle_s)
    steps, warmup = (max(2, args.steps // 10), 1) if large else (args.steps, args.warmup)
    say("prefill %s: warmup %d, steps %d" % (w.name, warmup, steps))
    wall_ms, ev_ms = leg.time_fwd(steps, warmup)
    split = leg.time_split(steps, warmup) if not large else None
    out["chunk16"], _ = leg_summary(leg, wall_ms, ev_ms, w.name + (", low-memory form" if low_memory else ""),
                                    split=split)
    out["device_error"] = leg.device_error()
    if idx == 1:
        del leg
        gc.collect()
        lg = PrefillLeg(dev, inp, chunk=64)
        wm, em = lg.time_fwd(args.steps, args.warmup)
        out["chunk64"], _ = leg_summary(lg, wm, em, w.name + ", chunk 64", C=64,
                                        split=lg.time_split(args.steps, args.warmup))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before each timed leg")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of back-to-back headline steps before the first timed leg (clock settle)")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-large", action="store_true", help="skip the 130K-token packed and 1M-token legs")
    ap.add_argument("--counters", action="store_true",
                    help="short pass for hardware-counter runs: a 1 GiB device copy (calibration of the byte "
                         "counters), then the prefill and decode steps, no CPU baseline")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two counter runs of --counters (FETCH_SIZE, WRITE_SIZE "
                         "run_counter_collection.csv) into per-kernel HBM bytes (profiles/traffic.json)")
    ap.add_argument("--mfma-from", metavar="SQ_CSV",
                    help="no GPU work: add SQ_VALU_MFMA_BUSY_CYCLES per launch from a counter run of --counters "
                         "(run_counter_collection.csv) to the counter summary (--traffic-out)")
    ap.add_argument("--traffic-out", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                          "traffic.json"))
    ap.add_argument("--config", type=int, choices=range(5), default=None,
                    help="time one workload only and print its JSON line: 0 tiny fp32 prefill (T=64, H=2, d=32), "
                         "1 prefill T=4096 H=96 d=128 bf16 (chunk 16 and 64), 2 16 packed sequences (~130K tokens), "
                         "3 decode N=512 H=96, 4 prefill T=1,048,576 H=96")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(*args.traffic_from, args.traffic_out)))
        if not args.mfma_from:
            return
    if args.mfma_from:
        print(json.dumps(mfma_from_counters(args.mfma_from, args.traffic_out)))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (heads and sequences would "
              "shard without communication; see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    def say(msg):
        print("[bench] " + msg, file=sys.stderr, flush=True)

    if args.config is not None:
        print(json.dumps(run_config(args.config, args, dev, say)), flush=True)
        return

    if args.counters:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        args.no_cpu_baseline = True
        args.no_large = True
        args.settle_s = 0.0
    w = synth.WORKLOADS["prefill_4k"]
    inp = synth.workload_prefill_inputs(w, device=dev)
    leg = PrefillLeg(dev, inp)
    settle = settle_clock(leg, args.settle_s) if args.settle_s > 0 else {"seconds": 0.0, "calls": 0}
    say("clock settled: %d headline steps in %.2f s; prefill %s: warmup %d, steps %d"
        % (settle["calls"], settle["seconds"], w.name, args.warmup, args.steps))
    wall_ms, ev_ms = leg.time_fwd(args.steps, args.warmup)
    prep_ms, state_ms = leg.time_split(args.steps, args.warmup)
    head, kb = leg_summary(leg, wall_ms, ev_ms, "", split=(prep_ms, state_ms))
    errors = {"prefill_4k": leg.device_error()}
    dom = "state" if state_ms >= prep_ms else "prep"
    dom_ms = state_ms if dom == "state" else prep_ms
    dom_gbs = kb[dom] / (dom_ms * 1e-3) / 1e9
    kname = "kda::kda_state_pass_fmt<128, 128>" if dom == "state" else "kda::kda_chunk_prep<true, 128, false, false>"
    out = {
        "metric": "KDA prefill tokens/s (H=96,d=128,bf16) + decode state GB/s, % of roofline",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,v~N(0,1), k L2-normalised, g=-5*sigmoid(N(0,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "prefill B=1 T=4096 H=96 K=V=128 bf16 chunk 16, zero S0, bf16 operands (default)",
                   "global_batch": 1, "seq_len": w.T, "heads": w.H, "chunk": 16, "parallelism": "single GPU"},
        "clock_settle": settle,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dom_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(kname),
                     "algorithmic_bytes_per_launch": kb[dom], "avg_launch_ms": dom_ms,
                     "mfma_busy_frac_rocprof": mfma_busy_frac(kname, dom_ms)},
        "roofline_path": head["roofline_path"],
        "event_ms_per_step": ev_ms,
        "kernels_ms": {"kda_chunk_prep (header + prep)": prep_ms, "kda_state_pass": state_ms},
        "split_calls_ms": prep_ms + state_ms,
        "workspace_bytes": leg.wsb,
    }
    del leg
    gc.collect()

    def prefill_leg(key, name, inp_, steps=args.steps, warmup=args.warmup, C=16, **kw):
        say("prefill %s: warmup %d, steps %d" % (key, warmup, steps))
        lg = PrefillLeg(dev, inp_, chunk=C, **kw)
        wm, em = lg.time_fwd(steps, warmup)
        sp = lg.time_split(steps, warmup) if lg.sws is not None else None
        out[key], _ = leg_summary(lg, wm, em, name, C=C, split=sp)
        errors[key] = lg.device_error()
        del lg
        gc.collect()  # the leg's closures refer back to it: free its buffers now
        torch.cuda.empty_cache()

    if not args.no_large:
        wv = synth.WORKLOADS["varlen_16"]
        inpv = synth.workload_prefill_inputs(wv, device=dev)
        T2 = inpv["q"].shape[1]
        prefill_leg("varlen_16", "16 packed sequences, lengths uniform in [256, 16384] (seed %d: %d tokens), "
                                 "H=96 K=V=128 bf16 chunk 16, S0 ~ N(0, 0.02^2), cu_seqlens" % (wv.seed, T2), inpv,
                    steps=max(3, args.steps // 4), warmup=2)
        del inpv
        w1 = synth.WORKLOADS["prefill_1m"]
        gc.collect()
        torch.cuda.empty_cache()
        free, _ = torch.cuda.mem_get_info()
        io_bytes = w1.T * w1.H * (3 * w1.K + 2 * w1.V + 1) * 2
        ws_bytes = _lib.load().kda_chunk_fwd_workspace_bytes(1, w1.T, w1.H, w1.K, w1.V, 1, 16, 1, 0, 0)
        inp1 = synth.workload_prefill_inputs(w1, device=dev)
        name1 = "B=1 T=1,048,576 H=96 K=V=128 bf16 chunk 16, zero S0"
        n1 = max(2, min(5, args.steps // 10))
        if free < io_bytes + ws_bytes + w1.H * w1.K * w1.V * 4 + (4 << 30):
            out["prefill_1m"] = {"skipped": "two passes need %.0f GB of device memory, %.0f GB free"
                                            % ((io_bytes + ws_bytes) / 1e9, free / 1e9)}
        else:
            prefill_leg("prefill_1m", name1 + ", two passes", inp1, steps=n1, warmup=1, with_split=False)
        torch.cuda.empty_cache()
        prefill_leg("prefill_1m_low_memory", name1 + ", low-memory form (one fused kernel)", inp1, steps=n1,
                    warmup=1, with_split=False, low_memory=True)
        del inp1
        torch.cuda.empty_cache()

    prefill_leg("chunk64", "prefill B=1 T=4096 H=96 K=V=128 bf16 chunk 64, zero S0", inp, C=64)
    prefill_leg("fp16_operands", "as the headline, fp16 state-pass operands (operands=fp16)", inp, operands="fp16")
    prefill_leg("low_memory", "as the headline, low-memory form (one fused kernel, workspace = header only)", inp,
                with_split=False, low_memory=True)
    del inp
    inp = synth.workload_prefill_inputs(w, device=dev, gate_preact=True)
    prefill_leg("gate_fused", "as the headline; g holds the gate pre-activation x, log-decay -5*sigmoid(x) formed "
                              "in-kernel", inp, gate="scaled_sigmoid")
    del inp
    inp = synth.workload_prefill_inputs(w, device=dev, gate_preact=True, with_o_gate=True)
    prefill_leg("gates_fused", "as gate_fused, plus an output gate: o * sigmoid(z), z [B,T,H,V] bf16 read and "
                               "applied where o is stored", inp, gate="scaled_sigmoid")
    del inp
    inp = synth.workload_prefill_inputs(w, device=dev, gate_preact=True, with_o_gate=True, raw_k=True)
    prefill_leg("prologue_epilogue_fused", "as gates_fused, with raw q, k ~ N(0,1) L2-normalised per (token, head) "
                                           "in-kernel", inp, gate="scaled_sigmoid", qk_norm=True)
    prefill_leg("conv_prologue_epilogue_fused", "as prologue_epilogue_fused, plus the length-4 short convolution of "
                                                "q, k, v with SiLU", inp, gate="scaled_sigmoid", qk_norm=True,
                conv="short4_silu")
    del inp
    if not args.no_decode:
        wd = synth.WORKLOADS["decode_512"]
        say("decode %s: %d steps" % (wd.name, args.decode_steps))
        d = time_decode(wd, args.decode_steps, dev)
        gbs = d["bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9
        out["decode"] = {"workload": "decode N=512 H=96 K=V=128 bf16 in, fp32 state in place, %d steps" %
                                     d["steps"],
                         "ms_per_step": d["ms_per_step"], "median_ms": d["median_ms"],
                         "tokens_per_s": d["N"] / (d["ms_per_step"] * 1e-3),
                         "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel", "achieved": gbs,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                      "traffic": measured_traffic("kda::kda_decode_kernel<true, 128, 128,"),
                                      "algorithmic_bytes_per_launch": d["bytes_per_step"]}}
        dg = time_decode(wd, args.decode_steps, dev, gate="scaled_sigmoid")
        out["decode"]["gate_fused_ms_per_step"] = dg["ms_per_step"]
        dn = time_decode(wd, args.decode_steps, dev, gate="scaled_sigmoid", qk_norm=True)
        out["decode"]["gate_and_qk_norm_fused_ms_per_step"] = dn["ms_per_step"]
        cp = time_copy(dev) if not args.counters else {"GB_per_s": float("nan")}
        out["hbm_copy_reference"] = dict(cp, what="torch device-to-device copy of 2 GiB: read + write bytes "
                                                  "per second, the rate a plain streaming kernel reaches")
        out["decode"]["frac_of_copy_rate"] = gbs / cp["GB_per_s"]
    if not args.no_backward:
        say("backward %s: warmup 3, steps 10" % w.name)
        rb = time_backward(w, 10, 3, dev)
        fl = backward_flops(rb["T"], rb["H"], rb["K"], rb["V"])
        tfs = fl / (rb["ms"] * 1e-3) / 1e12
        out["backward"] = {
            "workload": "kda_chunk_bwd on the prefill inputs (B=1 T=4096 H=96 K=V=128 bf16 in, fp32 gradients, "
                        "dL/do ~ N(0,1), no dL/dS_final)",
            "ms_per_step": rb["ms"], "tokens_per_s": rb["B"] * rb["T"] / (rb["ms"] * 1e-3),
            "workspace_bytes": rb["ws_bytes"],
            "roofline": {"bound": "mfma", "kernel": "kda_chunk_bwd (chunk factors, state pass, reverse pass, gradients)",
                         "achieved": tfs, "peak": FP32_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfs / FP32_MFMA_PEAK_TFS, "algorithmic_flops_per_call": fl,
                         "timed": "whole call (6 launches)"}}
        say("backward with the prologue (q/k norm, short convolution with SiLU): warmup 2, steps 5")
        rp = time_backward(w, 5, 2, dev, prologue=True)
        out["backward"]["with_prologue"] = {"ms_per_step": rp["ms"], "workspace_bytes": rp["ws_bytes"],
                                            "tokens_per_s": rp["B"] * rp["T"] / (rp["ms"] * 1e-3)}
        say("backward with an output gate: warmup 2, steps 5")
        rg = time_backward(w, 5, 2, dev, o_gate=True)
        out["backward"]["with_output_gate"] = {"ms_per_step": rg["ms"], "workspace_bytes": rg["ws_bytes"],
                                               "tokens_per_s": rg["B"] * rg["T"] / (rg["ms"] * 1e-3)}
        say("backward in 1024-token segments (workspace under 1 GB): warmup 2, steps 5")
        rs = time_backward(w, 5, 2, dev, segment_tokens=1024)
        out["backward"]["in_segments"] = {"ms_per_step": rs["ms"], "workspace_bytes": rs["ws_bytes"],
                                          "segment_tokens": 1024,
                                          "tokens_per_s": rs["B"] * rs["T"] / (rs["ms"] * 1e-3)}
    out["device_errors"] = errors
    if not args.no_cpu_baseline:
        say("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
