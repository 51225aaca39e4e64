"""Benchmark of the MI355X KDA hot path on one GPU; prints ONE JSON line.

A step is one chunked prefill (kda_chunk_prep + kda_chunk_state, i.e. one
kda_chunk_fwd) of the K3-shaped workload: B=1, T=4096, H=96, K=V=128, bf16
q/k/v/g/beta, chunk 16, zero initial state, returning o and S_final. Inputs
are seeded synthetic tensors already resident in HBM. `value` is prefill
tokens/s at chunk 16; the same workload is also timed at chunk 64 and
reported under "chunk64". The decode half of the metric (N=512 streams,
H=96, fp32 state of ~3.2 GB updated in place, 100 consecutive steps) is
timed after the prefill steps and reported under "decode". The backward pass
(kda_chunk_bwd) on the prefill workload's inputs is timed last and reported
under "backward", against the fp32 vector peak (it runs on the vector ALUs).

Kernel durations come from HIP events recorded on the stream the kernels run
on, around each phase of every timed step. Roofline figures use algorithmic
bytes (the tensors the operation must read and write once) divided by those
durations, against MI355X's published 8 TB/s HBM3E bandwidth.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

from kda_gated_delta_chunk_amd import _lib, decode_step, synth
from kda_gated_delta_chunk_amd.source_hash import csrc_hash

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 matrix, TFLOP/s
FP32_VECTOR_PEAK_TFS = 157.3    # MI355X fp32 vector, TFLOP/s
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


def time_prefill(w, steps, warmup, dev, chunk=16, gate="log_decay", o_gate=False, qk_norm=False, conv="none"):
    lib = _lib.load()
    gc = _lib.GATES[gate]
    qkc = _lib.KDA_QK_L2NORM if qk_norm else _lib.KDA_QK_AS_GIVEN
    inp = synth.workload_prefill_inputs(w, device=dev, gate_preact=(gate == "scaled_sigmoid"), with_o_gate=o_gate,
                                        raw_k=qk_norm)
    og = inp["o_gate"].data_ptr() if o_gate else None
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    N = B
    o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    Sf = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    cc = _lib.CONVS[conv]
    cw = None
    if conv != "none":
        cw = (0.5 * torch.randn((H, 2 * K + V, 4), generator=torch.Generator().manual_seed(7))).to(dev)
    wsb = lib.kda_chunk_fwd_workspace_bytes(B, T, H, K, V, N, chunk, 1, cc)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    p = {n: inp[n].data_ptr() for n in ("q", "k", "v", "g", "beta")}

    def prep():
        _lib.check(lib.kda_chunk_prep(p["q"], p["k"], p["g"], p["beta"], None, B, T, H, K, V, N, chunk, 1, gc, qkc,
                                      cc, None if cw is None else cw.data_ptr(), ws.data_ptr(), wsb, sh),
                   "kda_chunk_prep")

    def state():
        _lib.check(lib.kda_chunk_state(p["v"], og, None, None, B, T, H, K, V, N, chunk, 1, cc,
                                       None if cw is None else cw.data_ptr(), 1, o.data_ptr(), Sf.data_ptr(),
                                       ws.data_ptr(), wsb, sh), "kda_chunk_state")

    def fwd():
        _lib.check(lib.kda_chunk_fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], og, None, None, B, T, H, K, V, N, chunk,
                                     1, gc, qkc, cc, None if cw is None else cw.data_ptr(), 1, o.data_ptr(),
                                     Sf.data_ptr(), ws.data_ptr(), wsb, sh), "kda_chunk_fwd")

    # the step: one kda_chunk_fwd call (where the state pass leaves CUs free, the library runs the
    # prep of later chunks beside the state pass of earlier ones)
    for _ in range(warmup):
        fwd()
    evf = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evf[0].record(stream)
    for i in range(steps):
        fwd()
        evf[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = evf[0].elapsed_time(evf[steps]) / steps
    # per-kernel durations: the two halves as separate calls (kda_chunk_prep, kda_chunk_state)
    for _ in range(warmup):
        prep()
        state()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        prep()
        ev[i][1].record(stream)
        state()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    prep_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    state_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    return {"B": B, "T": T, "H": H, "K": K, "V": V, "N": N, "wall_s": wall, "fwd_ms": fwd_ms, "prep_ms": prep_ms,
            "state_ms": state_ms, "ws_bytes": wsb}


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


def backward_flops(T, H, K, V):
    """Flops of the per-token backward per call: one forward recompute (decay, read, write: 5KV) plus the
    reverse step (G += q do^T, S_t do, G^T k, beta G d - A dv, G - k dv^T, rowsum(GA * A), decay: 19KV)."""
    return 24 * K * V * T * H


def time_backward(w, steps, warmup, dev):
    """kda_chunk_bwd on the prefill workload's inputs, dL/do ~ N(0, 1), no dL/dS_final."""
    lib = _lib.load()
    inp = synth.workload_prefill_inputs(w, device=dev)
    B, T, H, K = inp["q"].shape
    V = inp["v"].shape[-1]
    do, _ = synth.output_grads(B, T, H, V, w.io, w.seed, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty((B, T, H, K), **f32) for _ in range(3)] + [torch.empty((B, T, H, V), **f32),
                                                                    torch.empty((B, T, H), **f32)]
    dq, dk, dg, dv, db = (t.data_ptr() for t in outs)
    dS0 = torch.empty((B, H, K, V), **f32)
    wsb = lib.kda_chunk_bwd_workspace_bytes(B, T, H, K, V, B)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    p = {n: inp[n].data_ptr() for n in ("q", "k", "v", "g", "beta")}

    def bwd():
        _lib.check(lib.kda_chunk_bwd(p["q"], p["k"], p["v"], p["g"], p["beta"], None, None, None, do.data_ptr(),
                                     None, B, T, H, K, V, B, 1, 0, dq, dk, dv, dg, db, None, dS0.data_ptr(),
                                     ws.data_ptr(), wsb,
                                     stream.cuda_stream), "kda_chunk_bwd")

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
    """Add each kda kernel's SQ_VALU_MFMA_BUSY_CYCLES per launch (average over its dispatches, summed
    over the device) from a rocprofv3 counter run of `bench.py --counters` to the counter summary,
    if that summary was taken on the same kernel sources."""
    import csv
    from collections import defaultdict
    with open(out_path) as fh:
        out = json.load(fh)
    if out.get("csrc_hash") != csrc_hash():
        raise SystemExit("%s was taken on other kernel sources; take FETCH_SIZE/WRITE_SIZE again first" % out_path)
    vals = defaultdict(list)
    for r in csv.DictReader(open(sq_csv)):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        if "kda" in name and r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
            vals[name].append(float(r["Counter_Value"]))
    for k, v in vals.items():
        out["kernels"].setdefault(k, {})["mfma_busy_cycles"] = sum(v) / len(v)
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
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        vals = defaultdict(list)
        for r in rows:
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if "kda" in name:
                vals[name].append(float(r["Counter_Value"]))
        return copy, {k: sum(v) / len(v) for k, v in vals.items()}

    fcopy, f = per_kernel(fetch_csv, "FETCH_SIZE")
    wcopy, w = per_kernel(write_csv, "WRITE_SIZE")
    fscale = copy_bytes / (fcopy * 1024.0)  # the copy reads and writes 1 GiB
    wscale = copy_bytes / (wcopy * 1024.0)
    out = {"csrc_hash": csrc_hash(), "fetch_scale": fscale, "write_scale": wscale, "kernels": {}}
    for k in sorted(set(f) | set(w)):
        fb = f.get(k, 0.0) * 1024.0 * fscale
        wb = w.get(k, 0.0) * 1024.0 * wscale
        out["kernels"][k] = {"fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb}
    with open(out_path, "w") as fh:
        fh.write(json.dumps(out, indent=1) + "\n")
    return out


def cpu_baseline(w):
    """The fp64 oracle on the host, on the full prefill workload (generation excluded)."""
    import oracle  # test infrastructure: only this baseline leg uses it
    inp = synth.workload_prefill_inputs(w, device="cpu")
    args = [inp[n] for n in ("q", "k", "v", "g", "beta")]
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    oracle.chunk_fwd(*args, threads=threads)
    dt = time.perf_counter() - t0
    B, T, H, _ = args[0].shape
    return {"value": B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "full workload: B=1 T=%d H=%d K=V=128 bf16 inputs, fp64 per-token recurrence, %.1f s" %
                      (T, H, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU clock needs some tens of milliseconds of load to settle")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
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
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(traffic_from_counters(*args.traffic_from, args.traffic_out)))
        if not args.mfma_from:
            return
    if args.mfma_from:
        print(json.dumps(mfma_from_counters(args.mfma_from, args.traffic_out)))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (heads and sequences would "
              "shard without communication; see the design notes). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.counters:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        args.no_cpu_baseline = True
    w = synth.WORKLOADS["prefill_4k"]
    print("[bench] prefill %s: warmup %d, steps %d" % (w.name, args.warmup, args.steps), file=sys.stderr,
          flush=True)
    r = time_prefill(w, args.steps, args.warmup, dev)
    ms = r["wall_s"] * 1e3 / args.steps
    tok_s = r["B"] * r["T"] / (ms * 1e-3)
    path_bytes, kb = prefill_algorithmic_bytes(r["T"] * r["B"], r["H"], r["K"], r["V"], r["N"])
    kern_ms = {"kda_chunk_prep (+chunk table)": r["prep_ms"], "kda_state_pass": r["state_ms"]}
    dom = "state" if r["state_ms"] >= r["prep_ms"] else "prep"
    dom_ms = r["state_ms"] if dom == "state" else r["prep_ms"]
    dom_gbs = kb[dom] / (dom_ms * 1e-3) / 1e9

    def path_roofline(rr, C):
        pm = rr["fwd_ms"]
        gbs = path_bytes / (pm * 1e-3) / 1e9
        tf = prefill_flops(rr["T"] * rr["B"], rr["H"], rr["K"], rr["V"], C) / (pm * 1e-3) / 1e12
        return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": path_bytes, "event_ms": pm, "mfma_tflops_algorithmic": tf,
                "mfma_frac_algorithmic": tf / BF16_PEAK_TFLOPS}

    out = {
        "metric": "KDA prefill tokens/s (H=96,d=128,bf16) + decode state GB/s, % of roofline",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,v~N(0,1), k L2-normalised, g=-5*sigmoid(N(0,1)), beta=sigmoid(N(0,1)))",
        "config": {"workload": "prefill B=1 T=4096 H=96 K=V=128 bf16 chunk 16, zero S0", "global_batch": 1,
                   "seq_len": r["T"], "heads": r["H"], "chunk": 16, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "kda_state_pass" if dom == "state" else "kda_chunk_prep",
                     "achieved": dom_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dom_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("kda::kda_state_pass<true, 128, 128, 1, false, true>" if dom == "state"
                                                 else "kda::kda_chunk_prep<true, 128, false, true>"),
                     "algorithmic_bytes_per_launch": kb[dom], "avg_launch_ms": dom_ms,
                     "mfma_busy_frac_rocprof": mfma_busy_frac("kda::kda_state_pass<true, 128, 128, 1, false, true>"
                                                              if dom == "state" else "kda::kda_chunk_prep<true, 128, false, true>",
                                                              dom_ms)},
        "roofline_path": path_roofline(r, 16),
        "kernels_ms": kern_ms,
        "kernels_mfma_busy_frac_rocprof": {
            "kda_chunk_prep": mfma_busy_frac("kda::kda_chunk_prep<true, 128, false, true>", r["prep_ms"]),
            "kda_state_pass": mfma_busy_frac("kda::kda_state_pass<true, 128, 128, 1, false, true>", r["state_ms"])},
        "split_calls_ms": r["prep_ms"] + r["state_ms"],
        "workspace_bytes": r["ws_bytes"],
    }
    print("[bench] prefill %s at chunk 64: warmup %d, steps %d" % (w.name, args.warmup, args.steps),
          file=sys.stderr, flush=True)
    r64 = time_prefill(w, args.steps, args.warmup, dev, chunk=64)
    ms64 = r64["wall_s"] * 1e3 / args.steps
    out["chunk64"] = {"workload": "prefill B=1 T=4096 H=96 K=V=128 bf16 chunk 64, zero S0",
                      "tokens_per_s": r64["B"] * r64["T"] / (ms64 * 1e-3), "ms_per_step": ms64,
                      "kernels_ms": {"kda_chunk_prep64 (+chunk table)": r64["prep_ms"],
                                     "kda_state_pass": r64["state_ms"]},
                      "split_calls_ms": r64["prep_ms"] + r64["state_ms"],
                      "roofline_path": path_roofline(r64, 64), "workspace_bytes": r64["ws_bytes"]}
    print("[bench] prefill %s with the gate formed in-kernel: warmup %d, steps %d" % (w.name, args.warmup,
                                                                                    args.steps),
          file=sys.stderr, flush=True)
    rg = time_prefill(w, args.steps, args.warmup, dev, gate="scaled_sigmoid")
    msg = rg["wall_s"] * 1e3 / args.steps
    out["gate_fused"] = {"workload": "prefill B=1 T=4096 H=96 K=V=128 bf16 chunk 16, zero S0; g holds the gate "
                                     "pre-activation x, log-decay -5*sigmoid(x) formed in kda_chunk_prep",
                         "tokens_per_s": rg["B"] * rg["T"] / (msg * 1e-3), "ms_per_step": msg,
                         "kernels_ms": {"kda_chunk_prep (+chunk table)": rg["prep_ms"],
                                        "kda_state_pass": rg["state_ms"]}}
    print("[bench] prefill %s with both gates formed in-kernel: warmup %d, steps %d" % (w.name, args.warmup,
                                                                                      args.steps),
          file=sys.stderr, flush=True)
    ro = time_prefill(w, args.steps, args.warmup, dev, gate="scaled_sigmoid", o_gate=True)
    mso = ro["wall_s"] * 1e3 / args.steps
    out["gates_fused"] = {"workload": "as gate_fused, plus an output gate: o * sigmoid(z), z [B,T,H,V] bf16 read "
                                      "and applied where kda_state_pass stores o",
                          "tokens_per_s": ro["B"] * ro["T"] / (mso * 1e-3), "ms_per_step": mso,
                          "kernels_ms": {"kda_chunk_prep (+chunk table)": ro["prep_ms"],
                                         "kda_state_pass": ro["state_ms"]}}
    print("[bench] prefill %s with both gates and the q/k normalisation in-kernel: warmup %d, steps %d"
          % (w.name, args.warmup, args.steps), file=sys.stderr, flush=True)
    rn = time_prefill(w, args.steps, args.warmup, dev, gate="scaled_sigmoid", o_gate=True, qk_norm=True)
    msn = rn["wall_s"] * 1e3 / args.steps
    print("[bench] prefill %s with the short convolution as well: warmup %d, steps %d"
          % (w.name, args.warmup, args.steps), file=sys.stderr, flush=True)
    rc = time_prefill(w, args.steps, args.warmup, dev, gate="scaled_sigmoid", o_gate=True, qk_norm=True,
                      conv="short4_silu")
    msc = rc["wall_s"] * 1e3 / args.steps
    out["conv_prologue_epilogue_fused"] = {
        "workload": "as prologue_epilogue_fused, plus the length-4 short convolution of q, k, v with SiLU "
                    "(q, k in kda_chunk_prep; v by kda_conv_v into the workspace)",
        "tokens_per_s": rc["B"] * rc["T"] / (msc * 1e-3), "ms_per_step": msc,
        "kernels_ms": {"kda_chunk_prep (+chunk table)": rc["prep_ms"],
                       "kda_conv_v + kda_state_pass": rc["state_ms"]}}
    out["prologue_epilogue_fused"] = {
        "workload": "as gates_fused, with raw q, k ~ N(0,1) L2-normalised per (token, head) in kda_chunk_prep",
        "tokens_per_s": rn["B"] * rn["T"] / (msn * 1e-3), "ms_per_step": msn,
        "kernels_ms": {"kda_chunk_prep (+chunk table)": rn["prep_ms"], "kda_state_pass": rn["state_ms"]}}
    if not args.no_decode:
        wd = synth.WORKLOADS["decode_512"]
        print("[bench] decode %s: %d steps" % (wd.name, args.decode_steps), file=sys.stderr, flush=True)
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
    if not args.no_backward:
        print("[bench] backward %s: warmup 3, steps 10" % w.name, file=sys.stderr, flush=True)
        rb = time_backward(w, 10, 3, dev)
        fl = backward_flops(rb["T"], rb["H"], rb["K"], rb["V"])
        tfs = fl / (rb["ms"] * 1e-3) / 1e12
        out["backward"] = {
            "workload": "kda_chunk_bwd on the prefill inputs (B=1 T=4096 H=96 K=V=128 bf16 in, fp32 gradients, "
                        "dL/do ~ N(0,1), no dL/dS_final)",
            "ms_per_step": rb["ms"], "tokens_per_s": rb["B"] * rb["T"] / (rb["ms"] * 1e-3),
            "workspace_bytes": rb["ws_bytes"],
            "roofline": {"bound": "alu", "kernel": "kda_chunk_bwd (checkpoint walk, reverse walk, tile sum)",
                         "achieved": tfs, "peak": FP32_VECTOR_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": tfs / FP32_VECTOR_PEAK_TFS, "algorithmic_flops_per_call": fl,
                         "timed": "whole call (3 launches)"}}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
