"""Throughput of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload causal8k]

One step = one forward (attn_fwd: online softmax, tau = 8 conditional
rescale, LSE) plus one backward (attn_bwd phases: D = rowsum(dO o O) and
LSE*log2 e, the key-block dK/dV kernel, the query-block dQ kernel) over one
batch of seeded synthetic bf16 inputs already resident in HBM. The backward
design is the library's default for the workload (at head_dim 128 and 256
the dK/dV kernel stores dS and the dQ kernel runs dQ = alpha dS K);
--bwd-recompute-dq, --bwd-store-ds and --bwd-fused-dq select one. Throughput
counts algorithmic flops: forward 4*B*H*Sq*Sk*d, backward 2.5x, both halved
for causal.

Prints one JSON line. The "roofline" object covers the dominant kernel (the
longest-running one; the dK/dV kernel for the fwd+bwd workloads), timed with
HIP events on the stream it runs on. "cpu_baseline" times the float64 oracle
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_causal8k.txt")


def sources_sha() -> str:
    """Hash of the kernel sources and build flags (identifies the measured build)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "exact_attention_71_amd")
    for f in sorted(glob.glob(os.path.join(pkg, "csrc", "*"))) + [os.path.join(pkg, "build.py")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, only when it was
    taken on these exact sources (else None)."""
    try:
        lines = open(TRAFFIC_FILE).read().split("\n")
    except OSError:
        return None
    sha = sources_sha()
    for ln in lines:
        f = dict(kv.split("=", 1) for kv in ln.split() if "=" in kv)
        if f.get("kernel") == kernel and f.get("workload") == workload and f.get("sources") == sha:
            return int(f["bytes"])
    return None


def stored_ds_read_bytes(w, lengths) -> int:
    """Algorithmic HBM bytes of the dQ kernel that reads the stored dS: every
    32 x 32 dS sub-tile with a visible (query, key) pair (2 KiB each) of every
    (sequence, query head), K read once per (sequence, KV head), dQ written."""
    seqs = lengths if w.varlen else [w.seqlen] * w.batch
    subtiles = 0
    for n in seqs:
        nq, nk = -(-n // 32), -(-n // 32)
        if w.causal:   # equal lengths: sub-tile (q, k) is visible iff k <= q
            subtiles += sum(min(q + 1, nk) for q in range(nq))
        else:
            subtiles += nq * nk
    tokens = sum(seqs)
    return (subtiles * w.heads_q * 2048 + tokens * w.heads_kv * w.head_dim * 2
            + tokens * w.heads_q * w.head_dim * 2)


def _describe(w) -> str:
    if w.varlen:
        return (f"{w.name}: {w.num_seqs} packed seqs len U[{w.len_lo},{w.len_hi}], Hq{w.heads_q} "
                f"Hkv{w.heads_kv} d{w.head_dim} {'causal' if w.causal else 'non-causal'} {w.passes}")
    return (f"{w.name}: B{w.batch} Hq{w.heads_q} Hkv{w.heads_kv} S{w.seqlen} d{w.head_dim} "
            f"{'causal' if w.causal else 'non-causal'} {w.passes}"
            + (" det" if w.deterministic else "") + (" QKx3 half heads" if w.scaled_heads else ""))


def device_info(torch) -> dict:
    """CU count and peak engine clock as the runtime reports them (clock via
    hipDeviceGetAttribute(hipDeviceAttributeClockRate = 5), in kHz)."""
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count}
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0 and val.value > 0:
            mhz = val.value / 1000.0
            out["peak_clock_mhz"] = mhz
            # dense bf16 MFMA: 4096 flop per CU per clock (1024 per SIMD)
            out["peak_bf16_tflops_at_clock"] = round(out["cus"] * 4096 * mhz * 1e6 / 1e12, 1)
            out["clock_source"] = "hipDeviceGetAttribute(ClockRate)"
    except OSError:  # pragma: no cover
        pass
    return out


def host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 20.0) -> dict:
    """Float64 oracle on a bounded sample: whole (sequence, head) slabs of the
    workload, fwd (+bwd), until about budget_s seconds have been spent."""
    import numpy as np
    import oracle
    from oracle.attention import head_backward, head_forward
    from workloads import draw_lengths, make_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    if w.varlen:
        lengths = draw_lengths(w.num_seqs, w.len_lo, w.len_hi, 71000 + w.number)
        sl = max(lengths)
    else:
        sl = w.seqlen
    # one batch row of the workload (all heads drawn, a few used), same distribution
    inp = make_inputs(1, sl, sl, w.heads_q, w.heads_kv, w.head_dim, seed=71000 + w.number,
                      scaled_heads=w.scaled_heads, with_grad=True)
    q, k, v, do = (oracle.attention._f64(inp[n])[0] for n in ("q", "k", "v", "do"))
    grp = w.heads_q // w.heads_kv
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    for h in range(w.heads_q):
        hk = h // grp
        head_forward(q[:, h], k[:, hk], v[:, hk], w.scale, w.causal)
        f = 4.0 * sl * sl * w.head_dim * (0.5 if w.causal else 1.0)
        flops += f
        if w.passes == "fwd+bwd":
            head_backward(q[:, h], k[:, hk], v[:, hk], do[:, h], w.scale, w.causal)
            flops += 2.5 * f
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"{heads} of {w.heads_q * (w.num_seqs if w.varlen else w.batch)} "
                      f"(sequence, head) slabs at length {sl}, {w.passes}, float64 numpy, "
                      f"{dt:.1f} s"}


def sweep_tau_exp(torch, ea, args) -> int:
    """Forward throughput vs the rescale threshold tau and the share of exp2
    evaluated on the FMA path (accuracy of the same settings against the
    oracle: tests/test_gpu_parity.py::test_tau_and_exp_emulation_variants_match_oracle)."""
    from workloads import Workload, workload_flops, workload_inputs
    for d in (64, 128, 256):
        w = Workload(f"sweep_d{d}", 6, 1, 8, 8, 16384, d, True, "fwd", scaled_heads=True)
        inp = workload_inputs(w, device="cuda:0")
        q, k, v = inp["q"], inp["k"], inp["v"]
        fl = workload_flops(w)["fwd"]
        o = torch.empty_like(q)
        lse = torch.empty((1, 8, 16384), dtype=torch.float32, device="cuda:0")
        for tau in (0, 4, 8, 16):
            for emu in (0, 1, 2, 4):
                ea.set_tuning("tau", tau)
                ea.set_tuning("exp_emulation", emu)
                for _ in range(args.warmup):
                    ea.fwd(q, k, v, causal=True, out=o, lse_out=lse)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                a.record()
                for _ in range(args.steps):
                    ea.fwd(q, k, v, causal=True, out=o, lse_out=lse)
                b.record()
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / args.steps
                print(json.dumps({"sweep": "tau_exp", "head_dim": d, "tau": tau, "exp_emulation": emu,
                                  "fwd_ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)}),
                      flush=True)
    ea.set_tuning("tau", 8)
    ea.set_tuning("exp_emulation", -1)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # steady state: the GPU's clocks ramp up over the first ~10 ms of sustained
    # MFMA load, so the default warmup covers about 50 ms of steps
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="causal8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--bwd-fused-dq", action="store_true",
                    help="time the fused backward (dQ atomics) instead of dK/dV + dQ kernels")
    ap.add_argument("--bwd-recompute-dq", action="store_true",
                    help="dQ kernel recomputing S and dP instead of reading the dS the dK/dV "
                         "kernel stores")
    ap.add_argument("--bwd-store-ds", action="store_true",
                    help="dQ from the dS the dK/dV kernel stores (fixed length)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: forward throughput over tau in {0,4,8,16} x "
                         "exp_emulation in {0,1,2,4} x d in {64,128,256} (B1 H8 S16384 causal, "
                         "Q,K x3 on half the heads), one JSON line per setting")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device 3 times (a known-size kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the attention path "
              "here has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import exact_attention_71_amd as ea
    from workloads import WORKLOADS, draw_lengths, workload_flops, workload_inputs

    w = WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.sweep:
        return sweep_tau_exp(torch, ea, args)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] workload {_describe(w)}", file=sys.stderr, flush=True)
    inp = workload_inputs(w, device=dev)
    lengths = draw_lengths(w.num_seqs, w.len_lo, w.len_hi, 71000 + w.number) if w.varlen else None
    fl = workload_flops(w, lengths)
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    with_bwd = w.passes == "fwd+bwd"

    if w.varlen:
        cu_q = inp["cu_seqlens_q"].to(dev)
        cu_k = inp["cu_seqlens_k"].to(dev)
        mx = max(lengths)
        tq, hq, d = q.shape
        p = ea.make_params(w.num_seqs, mx, mx, w.heads_q, w.heads_kv, d, w.scale, w.causal,
                           w.deterministic, total_q=tq, total_k=k.shape[0])
        o = torch.empty_like(q)
        lse = torch.empty((hq, tq), dtype=torch.float32, device=dev)
    else:
        cu_q = cu_k = None
        b, s, hq, d = q.shape
        p = ea.make_params(b, s, s, w.heads_q, w.heads_kv, d, w.scale, w.causal, w.deterministic)
        o = torch.empty_like(q)
        lse = torch.empty((b, hq, s), dtype=torch.float32, device=dev)
    varlen = w.varlen
    lib = ea.load()
    import ctypes
    if args.bwd_fused_dq:
        ea.set_tuning("bwd_fused_dq", 1)
    if args.bwd_store_ds:
        ea.set_tuning("bwd_store_ds", 1)
    if args.bwd_recompute_dq:
        ea.set_tuning("bwd_store_ds", 0)
    fused = ea.get_tuning("bwd_fused_dq")
    # the workspace size depends on the backward design (the stored dS lives there)
    stored_ds = ea.bwd_stores_ds(p, varlen) == 1
    fws = torch.empty(max(1, ea.fwd_workspace_size(p, varlen)), dtype=torch.uint8, device=dev)
    bws = torch.empty(max(1, ea.bwd_workspace_size(p, varlen)), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def run_fwd():
        st = stream()
        if varlen:
            r = lib.attn_fwd_varlen(ctypes.byref(p), cu_q.data_ptr(), cu_k.data_ptr(), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    fws.data_ptr(), fws.numel(), st)
        else:
            r = lib.attn_fwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), fws.data_ptr(), fws.numel(), st)
        assert r == 0, r

    def run_bwd_phase(mask):
        r = lib.attn_bwd_phases(ctypes.byref(p), None if cu_q is None else cu_q.data_ptr(),
                                None if cu_k is None else cu_k.data_ptr(), mask, q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                bws.data_ptr(), bws.numel(), stream())
        assert r == 0, r

    def stream():
        return torch.cuda.current_stream().cuda_stream

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # per-kernel HIP events on the launch stream: name -> list of (start, end)
    marks = {}

    def timed(name, fn, on):
        if not on:
            fn()
            return
        a, b = ev(), ev()
        a.record()
        fn()
        b.record()
        marks.setdefault(name, []).append((a, b))

    def step(on: bool):
        timed("fwd", run_fwd, on)
        if not with_bwd:
            return
        timed("bwd_pre", lambda: run_bwd_phase(ea.BWD_PREPROCESS), on)
        timed("bwd_main", lambda: run_bwd_phase(ea.BWD_MAIN), on)
        timed("bwd_dq", lambda: run_bwd_phase(ea.BWD_DQ), on)
        timed("bwd_post", lambda: run_bwd_phase(ea.BWD_POSTPROCESS), on)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step(True)
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    kms = {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in marks.items()}
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step; per kernel (ms): "
          + ", ".join(f"{n} {t:.3f}" for n, t in kms.items()), file=sys.stderr, flush=True)
    if with_bwd and w.deterministic:
        assert ea.bwd_status(p, bws, varlen) == 0

    # each public entry point as one ABI call (attn_fwd[_varlen]; attn_bwd[_varlen]
    # = every backward launch), hipEvent-timed on the stream, median and min
    def run_bwd_all():
        st = stream()
        if varlen:
            r = lib.attn_bwd_varlen(ctypes.byref(p), cu_q.data_ptr(), cu_k.data_ptr(), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    bws.data_ptr(), bws.numel(), st)
        else:
            r = lib.attn_bwd(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             bws.data_ptr(), bws.numel(), st)
        assert r == 0, r

    def abi_times(fn, n):
        ts = []
        for _ in range(n):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        ts.sort()
        return {"median": round(ts[len(ts) // 2], 4), "min": round(ts[0], 4), "calls": n}

    abi = {"attn_fwd" + ("_varlen" if varlen else ""): abi_times(run_fwd, 20)}
    if with_bwd:
        abi["attn_bwd" + ("_varlen" if varlen else "")] = abi_times(run_bwd_all, 20)

    total_flops = fl["fwd+bwd"] if with_bwd else fl["fwd"]
    value = total_flops / (ms * 1e-3) / 1e12
    # algorithmic flops per kernel: forward 2 GEMMs; the key-block backward kernel
    # S, dP, dV, dK (4 of the 5 backward GEMMs; all 5 when dQ is fused); the dQ
    # kernel only dQ (its recomputed S and dP are not algorithmic work)
    half = fl["fwd"] / 2.0
    kflops = {"fwd": fl["fwd"], "bwd_main": (5 if fused else 4) * half,
              "bwd_dq": 1 * half}
    names = {"fwd": f"fwd_kernel<{w.head_dim}>",
             "bwd_main": f"{'bwd_main' if fused else 'bwd_dkdv'}_kernel<{w.head_dim}>",
             "bwd_dq": f"bwd_dq_{'ds_' if stored_ds else ''}kernel<{w.head_dim}>"}
    dom = max((n for n in kms if n in kflops), key=lambda n: kms[n])
    dom_ms = kms[dom]
    dom_name = names[dom]
    achieved = kflops[dom] / (dom_ms * 1e-3) / 1e12
    kernels = {names[n]: {"ms": round(kms[n], 4),
                          "tflops": round(kflops[n] / (kms[n] * 1e-3) / 1e12, 1)}
               for n in kms if n in kflops and kms[n] > 0.002}
    if stored_ds and kms.get("bwd_dq", 0) > 0.002:
        # HBM-bound: its roofline is bandwidth, against the 8 TB/s peak
        b = stored_ds_read_bytes(w, lengths)
        gbs = b / (kms["bwd_dq"] * 1e-3) / 1e9
        kernels[names["bwd_dq"]].update({"bound": "hbm", "algorithmic_bytes": b,
                                         "gbs": round(gbs, 1),
                                         "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    out = {
        "metric": "attention fwd/bwd TFLOPs/s at hdim128 bf16; % of MI355X BF16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, resident in HBM)",
        "config": {"workload": _describe(w), "pass": w.passes,
                   "bwd_design": "fused dQ atomics" if fused else
                                 ("dK/dV kernel storing dS + dQ = dS K kernel" if stored_ds
                                  else "dK/dV kernel + dQ kernel recomputing S, dP"),
                   "kernels": kernels, "abi_ms": abi, "device": device_info(torch),
                   "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "kernel": dom_name,
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom_name, w.name),
                     "avg_launch_ms": round(dom_ms, 4), "sources": sources_sha()},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
