#!/usr/bin/env python3
"""Benchmark of the linear-attention hot path on one MI355X.

Default workload (the headline): causal linear attention, bf16 inputs with fp32
accumulation and state, B=2 H=16 N=32768 D=M=64 — one step is one full
``linattn_causal_fwd`` over the batch (every kernel of the causal path).
Other workloads (``--workload``): noncausal_long, decode (prefill + 1024
single-token steps on 256x16 states), deltanet, deltanet_decode (the same for the
delta-rule memory), softmax_decode (the same steps as softmax attention over a
key/value cache, the comparison baseline), fmap_dpfp1/2/3 and fmap_poly2 (causal
linear attention with the DPFP-nu or degree-2 polynomial feature map, fp32,
B=4 H=8 N=4096 D=M=64), causal_mid, causal_small, and copy (a 1 GiB device copy that calibrates
the HBM counters).

Prints ONE JSON line.  Inputs are synthetic (seeded N(0,1), the recipe of the
synth module), copied to the GPU before the timed region.  Timing: W untimed
warm-up steps, then K timed steps launched back to back and bracketed by a
device synchronisation; HIP events at both ends of the timed region are recorded
on the stream the library launches on (torch's current stream, passed to the C
ABI), and the average launch duration is the region over its launches.  Between
the W warm-up steps and the timed region, untimed steps run back to back for at
least --settle-ms (default 200 ms) whatever W is: the GPU's clocks ramp up under
sustained load, and the first ~100 launches of the causal kernel after idle run
up to 17% slower than the steady state.  The record states the settle phase
("settle"), and the median, minimum and maximum of individually timed launches
beside the mean ("launch_us").  The CPU baseline is the oracle timed on the host
cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector / matrix, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "causal linear-attn B·H·N tokens/s at N=32k, D=64; % of HBM/MFMA roofline"
PROFILE_DIR = os.path.join(ROOT, "profiles")


# Kernel sources each workload's launches are built from (the kernels and the
# headers they include): a counter summary is current while these are unchanged.
WORKLOAD_SOURCES = {
    "causal_long": ["causal_fused.hip", "lookback.hpp", "common.hpp", "lds_tiles.hpp"],
    "causal_mid": ["causal_fused32.hip", "lookback.hpp", "common.hpp", "lds_tiles.hpp"],
    "causal_bwd_long": ["causal_bwd.hip", "causal_bwd_bf16.hip", "causal.hip", "noncausal.hip", "common.hpp", "lds_tiles.hpp"],
    "noncausal_long": ["noncausal.hip", "common.hpp", "lds_tiles.hpp"],
    "decode": ["decode.hip", "common.hpp"],
    "deltanet": ["deltanet.hip", "deltanet_chunk.hip", "common.hpp"],
    "deltanet_decode": ["deltanet.hip", "common.hpp"],
    "softmax_decode": ["softmax_decode.hip", "common.hpp"],
    "fmap_dpfp1": ["featmap.hip", "causal.hip", "common.hpp"],
    "fmap_dpfp2": ["featmap.hip", "causal.hip", "common.hpp"],
    "fmap_dpfp3": ["featmap.hip", "causal.hip", "common.hpp"],
    "fmap_poly2": ["featmap.hip", "causal.hip", "common.hpp"],
}
# feature-map workloads: (linattn_fmap_t, nu)
FMAPS = {"fmap_dpfp1": (1, 1), "fmap_dpfp2": (1, 2), "fmap_dpfp3": (1, 3), "fmap_poly2": (2, 0)}


_CODE_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def code_text(src: str) -> str:
    """C++ source without its comments, with whitespace runs collapsed to one
    space (string and character literals kept as written)."""
    src = _CODE_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(src.split())


def source_hash(workload: str = None) -> str:
    """Hash of the kernel sources behind a workload (all of them without one),
    comments and layout ignored: counter figures taken from other code are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_recurrences_amd", "csrc")
    names = WORKLOAD_SOURCES.get(workload) or [n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp", ".cpp"))]
    for name in sorted(names):
        h.update(name.encode())
        h.update(code_text(open(os.path.join(csrc, name), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from a committed counter summary, if it matches the
    current kernel sources (else None).  The summary states FETCH/WRITE bytes per
    path launch already scaled by the copy-kernel calibration factor."""
    path = os.path.join(PROFILE_DIR, f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(workload):
        return None
    return float(m_bytes.group(1))


def mfma_from_profiles(workload: str):
    """MFMA busy fraction from a committed SQ counter summary, if it matches the
    current kernel sources (else None)."""
    path = os.path.join(PROFILE_DIR, f"{workload}_sq_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    m_busy = re.search(r"mfma_busy_frac:\s*([0-9.eE+-]+)", text)
    if not m_hash or not m_busy or m_hash.group(1) != source_hash(workload):
        return None
    return float(m_busy.group(1))


def runtime_info(torch) -> dict:
    """ROCm/HIP runtime and driver versions, the device and the host CPU."""
    import ctypes
    info = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
            "device": torch.cuda.get_device_name(0), "cpu_model": cpu_model(),
            "host_cores": len(os.sched_getaffinity(0))}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        for key, fn in (("hip_runtime_version", "hipRuntimeGetVersion"), ("hip_driver_version", "hipDriverGetVersion")):
            val = ctypes.c_int(0)
            if getattr(hip, fn)(ctypes.byref(val)) == 0:
                info[key] = val.value
    except OSError:
        pass
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    try:
        info["amdgpu_driver"] = open("/sys/module/amdgpu/version").read().strip()
    except OSError:
        pass
    return info


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_oracle(workload, inputs, budget_s: float = 20.0):
    """The oracle as it stands, on the host cores, on a bounded sample."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    w = workload
    if w.name == "decode" and len(inputs) == 6:
        q, k, v, sq, sk, sv = inputs
        nh = w.B * w.H
        # sample: all states, prefill + the first T steps
        t0 = time.perf_counter()
        _, S, z = oracle.causal(q, k, v, want_output=False)
        T = 0
        while T < w.steps:
            oracle.decode_step(sq[T], sk[T], sv[T], S, z)
            T += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        # prefill work counts as nh*N head-tokens, each step as nh head-tokens
        return {"value": nh * (w.N + T) / dt, "unit": "head-tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"prefill {w.N} tokens + {T} of {w.steps} steps on all {nh} states, {dt:.1f} s, "
                          f"{cpu_model()}"}
    if w.name == "fmap":  # another feature map: one head, then as many heads as the budget allows
        q, k, v, _, fm, nu = inputs
        omap = {1: oracle.DPFP, 2: oracle.POLY2}[fm]
        nh_all = w.B * w.H
        q, k, v = (t.reshape(1, nh_all, w.N, -1) for t in (q, k, v))
        t0 = time.perf_counter()
        oracle.fmap_causal(q[:, :1], k[:, :1], v[:, :1], omap, nu)
        one = time.perf_counter() - t0
        nh = max(1, min(nh_all, int(budget_s * threads / max(one, 1e-6))))
        nh = min(nh_all, max(threads, nh // threads * threads)) if nh >= threads else nh
        t0 = time.perf_counter()
        oracle.fmap_causal(q[:, :nh], k[:, :nh], v[:, :nh], omap, nu)
        dt = time.perf_counter() - t0
        return {"value": nh * w.N / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"{nh} of {nh_all} heads, all {w.N} tokens, {dt:.1f} s, {cpu_model()}"}
    if w.name == "causal_long" and len(inputs) == 4:  # backward: one head, then as many as the budget allows
        import torch
        from oracle import gradients
        q, k, v, dO = inputs
        t0 = time.perf_counter()
        gradients.causal_bwd(q[:1, :1], k[:1, :1], v[:1, :1], dO[:1, :1])
        one = time.perf_counter() - t0
        nh = max(1, min(w.B * w.H, int(budget_s / max(one, 1e-6))))
        qf, kf, vf, gf = (t.reshape(1, w.B * w.H, w.N, -1)[:, :nh] for t in (q, k, v, dO))
        t0 = time.perf_counter()
        gradients.causal_bwd(qf, kf, vf, gf)
        dt = time.perf_counter() - t0
        return {"value": nh * w.N / dt, "unit": "tokens/s", "cores": torch.get_num_threads(), "kind": "oracle",
                "sample": f"{nh} of {w.B * w.H} heads, all {w.N} tokens (fp64 autograd), {dt:.1f} s, {cpu_model()}"}
    if w.name == "decode" and len(inputs) == 7:  # softmax decode over the growing cache
        import numpy as np
        pq, pk, pv, sq, sk, sv, _ = inputs
        nh = w.B * w.H
        Lmax = w.N + w.steps
        Kc = np.zeros((w.B, w.H, Lmax, w.D))
        Vc = np.zeros((w.B, w.H, Lmax, w.M))
        Kc[:, :, :w.N] = oracle.f64(pk)
        Vc[:, :, :w.N] = oracle.f64(pv)
        t0 = time.perf_counter()
        T = 0
        while T < w.steps:
            _, Kc, Vc = oracle.softmax_decode(sq[T], sk[T], sv[T], Kc, Vc, w.N + T)
            T += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": nh * T / dt, "unit": "head-tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"the first {T} of {w.steps} steps (cache of {w.N}+ tokens) on all {nh} heads, {dt:.1f} s, "
                          f"{cpu_model()}"}
    if w.name == "deltanet_decode":
        q, k, v, beta, sq, sk, sv, sb = inputs
        nh = w.B * w.H
        # sample: all memories, prefill + the first T steps
        t0 = time.perf_counter()
        _, W = oracle.deltanet(q, k, v, beta)
        T = 0
        while T < w.steps:
            _, W = oracle.deltanet(sq[T][:, :, None], sk[T][:, :, None], sv[T][:, :, None], sb[T][:, :, None], W0=W)
            T += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": nh * (w.N + T) / dt, "unit": "head-tokens/s", "cores": threads, "kind": "oracle",
                "sample": f"prefill {w.N} tokens + {T} of {w.steps} steps on all {nh} memories, {dt:.1f} s, "
                          f"{cpu_model()}"}
    heads = w.B * w.H
    if w.name == "deltanet":
        q, k, v, beta = inputs
    else:
        q, k, v = inputs[:3]
    # time one head first, then choose the sample size from it
    t0 = time.perf_counter()
    if w.name == "deltanet":
        oracle.deltanet(q[:1, :1], k[:1, :1], v[:1, :1], beta[:1, :1])
    elif w.name.startswith("noncausal"):
        oracle.noncausal(q[:1, :1], k[:1, :1], v[:1, :1])
    else:
        oracle.causal(q[:1, :1], k[:1, :1], v[:1, :1])
    one = time.perf_counter() - t0
    nb = max(1, min(w.B, int(budget_s / max(one * w.H / threads, 1e-6))))
    t0 = time.perf_counter()
    if w.name == "deltanet":
        oracle.deltanet(q[:nb], k[:nb], v[:nb], beta[:nb])
    elif w.name.startswith("noncausal"):
        oracle.noncausal(q[:nb], k[:nb], v[:nb])
    else:
        oracle.causal(q[:nb], k[:nb], v[:nb])
    dt = time.perf_counter() - t0
    toks = nb * w.H * w.N
    return {"value": toks / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_thread": {"value": w.N / one, "unit": "tokens/s", "sample": "one head on one thread"},
            "sample": f"{nb} of {w.B} batch entries ({nb * w.H} of {heads} heads, all {w.N} tokens), "
                      f"{dt:.1f} s, {cpu_model()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default per workload: 100 for the sequence workloads, 20 for decode, "
                         "5 for softmax_decode)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default per workload: enough back-to-back work, >= 50 ms, for "
                         "the GPU's clocks to settle; a few launches after idle run up to 15%% slower)")
    ap.add_argument("--workload", default="causal_long",
                    choices=["causal_long", "causal_bwd_long", "noncausal_long", "decode", "deltanet", "deltanet_decode",
                             "softmax_decode", *FMAPS,
                             "causal_mid", "causal_small", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", nargs="?", const="read", choices=["read", "write"], default=None,
                    help="cold caches: before every launch, read (default) or write a 1 GiB buffer, and time each "
                         "launch with its own events (the default times back-to-back launches).  A read evicts the "
                         "L2s and the Infinity Cache without leaving dirty lines; after a write, the launch also pays "
                         "the write-back of the lines it evicts")
    ap.add_argument("--oracle-budget", type=float, default=20.0)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed back-to-back steps after the warm-up, at least this long, so that the timed "
                         "region runs at settled clocks whatever --warmup is")
    args = ap.parse_args()

    long_steps = {"decode": (20, 5), "deltanet_decode": (20, 5), "softmax_decode": (5, 2), "copy": (20, 5)}
    d_steps, d_warm = long_steps.get(args.workload, (100, 300))
    if args.steps is None:
        args.steps = d_steps
    if args.warmup is None:
        args.warmup = d_warm

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the per-(batch, head) problems shard across GPUs without communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import weight_recurrences_amd as la

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(3)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.workload == "copy":
        # Calibration: a plain 1 GiB device copy (torch's copy kernel).  Its
        # FETCH_SIZE / WRITE_SIZE counter readings against the known 1 GiB give
        # the factors that turn those counters into HBM bytes.
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        print(json.dumps({"metric": "device copy GB/s (read + write)", "value": 2 * nbytes / (ms / 1e3) / 1e9,
                          "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": ms, "higher_is_better": True, "bytes_per_copy": nbytes}), flush=True)
        return

    wname = {"noncausal_long": "causal_long", "causal_bwd_long": "causal_long",
             "softmax_decode": "decode", **{f: "fmap" for f in FMAPS}}.get(args.workload, args.workload)
    w = synth.WORKLOADS[wname]
    inputs = synth.workload_inputs(w)
    K, Wm = args.steps, args.warmup

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    if args.workload in ("causal_long", "causal_mid", "causal_small", "noncausal_long"):
        q, k, v = (t.to(dev) for t in inputs)
        o = torch.empty(w.B, w.H, w.N, w.M, dtype=w.dtype, device=dev)
        if args.workload == "noncausal_long":
            ws = torch.empty(max(1, la.noncausal_workspace_bytes(w.B, w.H, w.N, w.D, w.M, w.dtype)),
                             dtype=torch.uint8, device=dev)
            step = lambda: la.noncausal(q, k, v, out=o, workspace=ws)
            kernel = "linattn_noncausal_fwd (nc_state_kernel + nc_reduce_kernel + nc_apply_kernel)"
        else:
            ws = torch.empty(max(1, la.causal_workspace_bytes(w.B, w.H, w.N, w.D, w.M, w.dtype)),
                             dtype=torch.uint8, device=dev)
            step = lambda: la.causal(q, k, v, out=o, workspace=ws)
            kernel = ("causal_fused_kernel (single pass)" if w.dtype == torch.bfloat16 else "causal_fused32_kernel (single pass)")
        units = w.B * w.H * w.N                      # tokens per step
        es = torch.tensor([], dtype=w.dtype).element_size()
        alg_bytes = units * (2 * w.D + 2 * w.M) * es  # read q, k, v; write o
        unit = "tokens/s"
        launches_per_step = 1
    elif args.workload in FMAPS:
        fm, nu = FMAPS[args.workload]
        q, k, v = (t.to(dev) for t in inputs)
        o = torch.empty(w.B, w.H, w.N, w.M, dtype=w.dtype, device=dev)
        ws = torch.empty(max(1, la.fmap_workspace_bytes(w.B, w.H, w.N, w.D, w.M, w.dtype, fm, nu)),
                         dtype=torch.uint8, device=dev)
        step = lambda: la.fmap(q, k, v, fm, nu, out=o, workspace=ws)
        kernel = "linattn_fmap_fwd (fm_state_kernel + state_scan_kernel + fm_out_kernel)"
        units = w.B * w.H * w.N
        alg_bytes = units * (2 * w.D + 2 * w.M) * 4
        unit = "tokens/s"
        launches_per_step = 1
    elif args.workload == "causal_bwd_long":
        q, k, v = (t.to(dev) for t in inputs)
        dO = synth.qkv(w.B, w.H, w.N, w.M, w.M, dtype=w.dtype, seed=w.seed + 50)[0].to(dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(max(1, la.causal_bwd_workspace_bytes(w.B, w.H, w.N, w.D, w.M, w.dtype)), dtype=torch.uint8,
                         device=dev)
        step = lambda: la.causal_bwd(q, k, v, dO, out=grads, workspace=ws)
        kernel = ("linattn_causal_bwd (nc_state (block increments) + state_scan + bwd_q + bwd_rstate + suffix_scan + bwd_kv "
                  "kernels)")
        units = w.B * w.H * w.N
        es = 2
        alg_bytes = units * (4 * w.D + 3 * w.M) * es  # read q, k, v, dO; write dq, dk, dv
        unit = "tokens/s"
        launches_per_step = 1
        inputs = (inputs[0], inputs[1], inputs[2], dO.cpu())
    elif args.workload == "decode":
        pq, pk, pv, sq, sk, sv = inputs
        pq, pk, pv = pq.to(dev), pk.to(dev), pv.to(dev)
        sq, sk, sv = sq.to(dev), sk.to(dev), sv.to(dev)
        S0, z0 = la.causal(pq, pk, pv, output=False)
        S, z = S0.clone(), z0.clone()
        o = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=dev)

        def launch(t):
            la.decode_step(sq[t], sk[t], sv[t], S, z, out=o[t])

        def step():
            for t in range(w.steps):
                launch(t)
        kernel = "linattn_decode_step (decode_step_kernel)"
        units = w.B * w.H * w.steps                  # head-tokens per step (1024 decode steps)
        es = 2
        per_head_token = 2 * w.D * w.M * 4 + 2 * w.D * 4 + (2 * w.D + 2 * w.M) * es
        alg_bytes = w.B * w.H * per_head_token       # per launch (one decode step)
        unit = "head-tokens/s"
        launches_per_step = w.steps
    elif args.workload == "softmax_decode":
        # The decode workload's inputs: its 512 prefill tokens fill the key/value
        # cache, then each of the 1024 steps appends one token and attends over
        # the whole cache (L = 512 .. 1535).
        pq, pk, pv, sq, sk, sv = inputs
        Lmax = w.N + w.steps
        Kc = torch.zeros(w.B, w.H, Lmax, w.D, dtype=w.dtype, device=dev)
        Vc = torch.zeros(w.B, w.H, Lmax, w.M, dtype=w.dtype, device=dev)
        Kc[:, :, :w.N] = pk.to(dev)
        Vc[:, :, :w.N] = pv.to(dev)
        sq, sk, sv = sq.to(dev), sk.to(dev), sv.to(dev)
        o = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=dev)

        def launch(t):
            la.softmax_decode_step(sq[t], sk[t], sv[t], Kc, Vc, w.N + t, out=o[t])

        def step():
            for t in range(w.steps):
                launch(t)
        kernel = "softmax_decode_step (softmax_decode_kernel)"
        units = w.B * w.H * w.steps
        es = 2
        # per head and step: read the L cached rows and q, k, v; write row L and o
        rows = sum(w.N + t for t in range(w.steps)) / w.steps
        per_head_step = (rows * (w.D + w.M) + 2 * w.D + 2 * w.M + (w.D + w.M)) * es
        alg_bytes = int(w.B * w.H * per_head_step)   # per launch, averaged over the 1024 steps
        unit = "head-tokens/s"
        launches_per_step = w.steps

        # the linear decode step on the same inputs, for the ratio
        S0, z0 = la.causal(pq.to(dev), pk.to(dev), pv.to(dev), output=False)
        S, z = S0.clone(), z0.clone()
        ol = torch.empty_like(o)

        def linear_step():
            for t in range(w.steps):
                la.decode_step(sq[t], sk[t], sv[t], S, z, out=ol[t])
    elif args.workload == "deltanet_decode":
        q, k, v, beta, sq, sk, sv, sb = inputs
        q, k, v, beta = q.to(dev), k.to(dev), v.to(dev), beta.to(dev)
        sq, sk, sv, sb = sq.to(dev), sk.to(dev), sv.to(dev), sb.to(dev)
        _, W0 = la.deltanet(q, k, v, beta, return_state=True)
        W = W0.clone()
        o = torch.empty(w.steps, w.B, w.H, w.M, dtype=w.dtype, device=dev)

        def launch(t):
            la.deltanet_decode_step(sq[t], sk[t], sv[t], sb[t], W, out=o[t])

        def step():
            for t in range(w.steps):
                launch(t)
        kernel = "deltanet_decode_step (deltanet_step_kernel)"
        units = w.B * w.H * w.steps                  # head-tokens per step (1024 decode steps)
        es = 2
        per_head_token = 2 * w.M * w.D * 4 + (2 * w.D + 2 * w.M) * es + es
        alg_bytes = w.B * w.H * per_head_token       # per launch (one decode step)
        unit = "head-tokens/s"
        launches_per_step = w.steps
    else:  # deltanet
        q, k, v, beta = (t.to(dev) for t in inputs)
        o = torch.empty(w.B, w.H, w.N, w.M, dtype=w.dtype, device=dev)
        ws = torch.empty(max(1, la.deltanet_workspace_bytes(w.B, w.H, w.N, w.D, w.M, w.dtype)), dtype=torch.uint8,
                         device=dev)
        step = lambda: la.deltanet(q, k, v, beta, out=o, workspace=ws)
        kernel = "deltanet_fwd (dn_prep_kernel + dn_scan_kernel + dn_out_kernel)"
        units = w.B * w.H * w.N
        alg_bytes = units * ((2 * w.D + 2 * w.M) * 4 + 4)
        unit = "tokens/s"
        launches_per_step = 1

    if launches_per_step == 1:
        launch = lambda t: step()

    for _ in range(Wm):
        step()
    torch.cuda.synchronize()

    # Clock settle: untimed steps back to back for at least --settle-ms of wall
    # time (synchronising every few steps keeps the host close to the device).
    settle_steps = 0
    settle0 = time.perf_counter()
    if not args.flush:
        while (time.perf_counter() - settle0) * 1e3 < args.settle_ms:
            step()
            settle_steps += 1
            if settle_steps % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - settle0) * 1e3

    # Timed region: K steps launched back to back on the library's stream, HIP
    # events at both ends.  The average launch duration is the region's time over
    # the launches in it (the launches queue without host gaps, so this matches
    # the kernel trace's per-dispatch average).
    t_start, t_end = events(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if args.flush:
        # Cold caches: a 1 GiB buffer (4x the Infinity Cache, 32x the L2s) is
        # read (summed) before every launch, outside the launch's own pair of
        # events; the time is the sum of the launches' intervals.  Reading
        # leaves only clean lines in the caches; "write" fills the buffer
        # instead, and the next launch then also pays the write-back of the
        # dirty lines it evicts.
        flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        flush_out = torch.empty((), dtype=torch.float32, device=dev)

        def flush():
            if args.flush == "write":
                flush_buf.fill_(1.0)
            else:
                torch.sum(flush_buf, dim=0, out=flush_out)
        flush()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(K):
            for t in range(launches_per_step):
                flush()
                a, b = events(2)
                a.record(stream)
                launch(t)
                b.record(stream)
                pairs.append((a, b))
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = sum(a.elapsed_time(b) for a, b in pairs)
    else:
        t_start.record(stream)
        for _ in range(K):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_start.elapsed_time(t_end)
    launch_ms = total_ms / (K * launches_per_step)

    # Individually timed launches (after the timed region, same settled state):
    # each launch between its own pair of events, for the median, min and max
    # beside the mean of the back-to-back region.
    n_single = min(K * launches_per_step, 512)
    singles = []
    for i in range(n_single):
        a, b = events(2)
        if args.flush:
            flush()
        a.record(stream)
        launch(i % launches_per_step)
        b.record(stream)
        singles.append((a, b))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in singles)
    launch_us = {"mean_back_to_back": round(launch_ms * 1e3, 2), "median": round(us[len(us) // 2], 2),
                 "min": round(us[0], 2), "max": round(us[-1], 2), "n": len(us),
                 "note": "median/min/max of launches timed one by one with their own events"}

    ms_per_step = total_ms / K
    value = units * K / (total_ms / 1e3)
    achieved = alg_bytes / (launch_ms / 1e3) / 1e9
    traffic = traffic_from_profiles(args.workload)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "algorithmic_bytes_per_launch": alg_bytes, "launch_ms": round(launch_ms, 5)}
    if args.workload == "softmax_decode" and not args.flush:
        for _ in range(Wm):
            linear_step()
        a, b = events(2)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(K):
            linear_step()
        b.record(stream)
        torch.cuda.synchronize()
        lin_ms = a.elapsed_time(b) / K
        roofline["linear_decode_same_inputs"] = {"ms_per_step": round(lin_ms, 4),
                                                  "softmax_over_linear_time": round(ms_per_step / lin_ms, 2)}
    if args.workload in FMAPS:
        # The recurrent form's arithmetic with C features: S update 2CM, numerator
        # 2CM, z C, denominator 2C, the map itself C.  fp32 matrix work dominates.
        # The degree-2 polynomial map is defined with D^2 features, but x_a x_b =
        # x_b x_a leaves D (D + 1) / 2 distinct ones: `frac` counts those (the
        # minimal exact map); the kernels carry the pairs a <= b in groups of 16
        # (16 * 8 (D/16) (D/16 + 1) features), reported beside it with the defined
        # count.  DPFP's 2 nu D features are all distinct.
        C = la.fmap_dim(fm, nu, w.D)
        if fm == la.FMAP_POLY2:
            c_min, c_exec = w.D * (w.D + 1) // 2, 16 * 8 * (w.D // 16) * (w.D // 16 + 1)
        else:
            c_min = c_exec = C
        fl = lambda c: units * (4 * c * w.M + 4 * c)
        flops = fl(c_min)
        tfl = lambda c: fl(c) / (launch_ms / 1e3) / 1e12
        tflops = tfl(c_min)
        bf16_tflops = 3 * units * 4 * c_exec * w.M / (launch_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / FP32_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": kernel,
                    "algorithmic_flops_per_launch": flops, "feature_dim": c_min, "launch_ms": round(launch_ms, 5),
                    "feature_dims": {"minimal_exact": c_min, "executed": c_exec, "defined": C},
                    "frac_executed": round(tfl(c_exec) / FP32_PEAK_TFLOPS, 4),
                    "frac_defined": round(tfl(C) / FP32_PEAK_TFLOPS, 4),
                    # The state and output products run as three bf16 MFMAs each
                    # (head x head, head x tail, tail x head) over the executed
                    # features: the matrix units' own measure of the same launch.
                    "bf16_mfma": {"executed_tflops": round(bf16_tflops, 3), "peak": BF16_PEAK_TFLOPS,
                                  "frac": round(bf16_tflops / BF16_PEAK_TFLOPS, 4)},
                    "hbm": {"achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                            "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": alg_bytes}}
    if args.workload == "deltanet":
        flops = units * (6 * w.D * w.M + 6 * w.D)
        roofline["alu"] = {"achieved_tflops": round(flops / (launch_ms / 1e3) / 1e12, 3),
                           "peak_tflops": FP32_PEAK_TFLOPS}

    cpu = None
    if not args.no_cpu_baseline:
        extra = ("softmax",) if args.workload == "softmax_decode" else ()
        if args.workload in FMAPS:
            extra = ("fmap",) + FMAPS[args.workload]
        cpu = time_oracle(w, tuple(inputs) + extra, args.oracle_budget)

    names = {
        "causal_long": f"causal_long: causal linear attention (phi=elu+1), bf16 in/out, fp32 state, "
                       f"B={w.B} H={w.H} N={w.N} D=M={w.D}",
        "noncausal_long": f"noncausal_long: non-causal linear attention, bf16, B={w.B} H={w.H} N={w.N} D=M={w.D}",
        "causal_mid": f"causal_mid: causal linear attention, fp32, B={w.B} H={w.H} N={w.N} D=M={w.D}",
        "causal_small": f"causal_small: causal linear attention, fp32, B={w.B} H={w.H} N={w.N} D=M={w.D} (launch-bound)",
        "causal_bwd_long": f"causal_bwd_long: backward of causal linear attention (dq, dk, dv), bf16 in/out, fp32 "
                           f"arithmetic, B={w.B} H={w.H} N={w.N} D=M={w.D}",
        "decode": f"decode: RNN-form decode, {w.B}x{w.H} states D=M={w.D}, {w.steps} single-token bf16 steps "
                  f"after a {w.N}-token prefill",
        "deltanet": f"deltanet: delta-rule fast weights, fp32, B={w.B} H={w.H} N={w.N} D=M={w.D}",
        "deltanet_decode": f"deltanet_decode: delta-rule decode, {w.B}x{w.H} memories D=M={w.D}, {w.steps} "
                           f"single-token bf16 steps after a {w.N}-token prefill",
        "softmax_decode": f"softmax_decode: softmax attention decode over a key/value cache (comparison baseline), "
                          f"{w.B}x{w.H} heads D=M={w.D}, {w.steps} single-token bf16 steps after a {w.N}-token cache",
        **{f: f"{f}: causal linear attention with the "
              f"{'DPFP-%d' % FMAPS[f][1] if FMAPS[f][0] == 1 else 'degree-2 polynomial'} feature map "
              f"(C={la.fmap_dim(*FMAPS[f], w.D)}), fp32, B={w.B} H={w.H} N={w.N} D=M={w.D}" for f in FMAPS},
    }
    dtype = {"causal_long": "bf16", "causal_bwd_long": "bf16", "noncausal_long": "bf16", "decode": "bf16", "causal_mid": "f32", "causal_small": "f32",
             "deltanet": "f32", "deltanet_decode": "bf16", "softmax_decode": "bf16",
             **{f: "f32" for f in FMAPS}}[args.workload]
    if traffic is not None:
        # The HBM bytes the counters measured, moved in the measured launch time:
        # how close the path runs to the memory system on the bytes it really
        # moves (against `achieved`, which counts only the algorithmic ones).
        tr = traffic / (launch_ms / 1e3) / 1e9
        roofline["traffic_rate"] = {"achieved": round(tr, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(tr / HBM_PEAK_GBS, 4)}
    line = {
        "metric": METRIC if args.workload == "causal_long" else f"{args.workload} {unit}",
        "value": value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded N(0,1) inputs; no datasets or trained weights)",
        "config": {"workload": names[args.workload], "B": w.B, "H": w.H, "N": w.N, "D": w.D, "M": w.M,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "timing": (f"cold: 1 GiB {'read' if args.flush == 'read' else 'written'} before every launch, per-launch "
                   "events summed" if args.flush else "back-to-back launches between two events"),
        "cpu_baseline": cpu,
        "launch_us": launch_us,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "note": "untimed back-to-back steps between the warm-up and the timed region"},
        "mfma_busy_frac": mfma_from_profiles(args.workload),
        "env": runtime_info(torch),
        "wall_s": round(wall, 4),
        "source_hash": source_hash(args.workload),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
