"""Throughput of the Titans memory scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one titans_mem_scan call over the whole workload (every batch row
and head, all T tokens), with inputs already resident in HBM.  Prints ONE JSON
line.  value = tokens/s = B*T / (seconds per step).

roofline: algorithmic flops per launch of the scan kernel -- per token-head
    12 P - 2 n_1 n_0 + (C - 1) sum_l (n_{l-1} + n_l)
(key forward 2P, backward 2(P - n_1 n_0), reads at the in-chunk weights 4P,
chunk-end carry of theta and s 4P, strictly-lower C x C decay-masked terms)
-- divided by the kernel's average duration from HIP events recorded on the
stream the kernel runs on, against the MI355X peak of the unit that executes
it.
cpu_baseline: the fp64 oracle on a bounded sample of the same workload (the first
batch rows, every head, all or a prefix of the tokens) on the host cores.
retrieve: titans_mem_retrieve over the same q with the scan's final weights.
biases: the same scan with the Huber (delta 0.5) and l_p (p 3) attentional biases.
surprise: titans_mem_scan_surprise (the scan plus each token's gradient norm).
backward: titans_mem_scan_backward (cotangents of every input for seeded output
cotangents) on the same inputs, with its own roofline: the products of the checkpointing
forward sweep and the reverse chunk loop (bwd_alg_flops_per_token_head) on the fp32
matrix cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "memory-scan tokens/sec at 16 heads×d64, T=16K; % of MFMA/HBM roofline"

PEAKS = {  # MI355X published dense peaks
    "mfma_bf16": 2500.0,   # TFLOP/s
    "mfma_f32": 157.3,
    "valu_f32": 157.3,
    "hbm": 8000.0,         # GB/s
    "valu_slots": 78.64,   # T lane-slots/s: 256 CUs x 4 SIMDs x 32 fp32 lanes x 2.4 GHz
                           # (157.3 TFLOP/s counts an FMA as two flops)
}


def alg_flops_per_token_head(widths, C):
    P = sum(widths[l] * widths[l - 1] for l in range(1, len(widths)))
    lower = (C - 1) * sum(widths[l - 1] + widths[l] for l in range(1, len(widths)))
    return 12 * P - 2 * widths[1] * widths[0] + lower


def bwd_alg_flops_per_token_head(widths, C):
    """Products of the reverse pass per token-head, checkpointing forward sweep included.
    Per layer l (P_l = n_l n_{l-1}), 2 P_l flops per token for each of: the sweep's key
    forward, key backward (l >= 2) and two carries; the recompute's key forward, key backward
    (l >= 2) and two in-chunk read products (l < L); the query adjoint's two products with
    W_l, S_l; the chunk-end products with the two state cotangents; the key tangent
    product (l >= 2); the tangent backward's three products; the state-cotangent carry's
    three products plus one (l >= 2) -- 14 + 4 [l >= 2] + 2 [l < L] in all.  Plus the
    strictly-lower C x C terms, (C - 1)(3 n_{l-1} + 2 n_l + n_l [l < L]) per token, and three
    P-long dot products per chunk."""
    L = len(widths) - 1
    P = sum(widths[l] * widths[l - 1] for l in range(1, L + 1))
    total = 6.0 * P / C
    for l in range(1, L + 1):
        nin, nout = widths[l - 1], widths[l]
        units = 14 + 4 * (l >= 2) + 2 * (l < L)
        total += units * 2 * nin * nout + (C - 1) * (3 * nin + 2 * nout + nout * (l < L))
    return total


def alg_bytes(wl):
    """q, k, v, y once; three fp32 gates; theta0, s0 in and theta_T, s_T out once per memory."""
    io = 2 if wl.io == "bf16" else 4
    th = wl.batch * wl.seq_len * wl.heads
    return th * (4 * wl.d * io + 12) + 4 * 4 * wl.params * wl.batch * wl.heads


# the kernels of one titans_mem_scan call, by path family
KERNELS = {
    "fused": "scan_mfma_kernel",
    "generic": "scan_generic_kernel",
    "phased": "phase_kernel",
    "linear": "linear_summary_kernel + linear_combine_kernel + scan_generic_kernel",
}


def kernel_source_digest(kernel):
    """sha256 of the source file that defines the kernel (traffic is void once it changes)."""
    import hashlib

    src = ("scan_pair.hip" if "scan_pair_kernel" in kernel else
           "scan_mfma.hip" if "scan_mfma_kernel" in kernel else
           "scan_phased.hip" if "phase_kernel" in kernel else "scan_generic.hip")
    with open(os.path.join(ROOT, "sequence_models_amd", "csrc", src), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the stored rocprofv3 FETCH_SIZE / WRITE_SIZE runs, each
    scaled by what the counter read for a plain copy of known size; None if the kernel
    source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha256") != kernel_source_digest(kernel):
        return None
    return rec["fetch_kib"] * 1024 * rec["fetch_scale"] + rec["write_kib"] * 1024 * rec["write_scale"]


def cpu_baseline(inp, wl, sample_rows, sample_tokens, single_tokens=1024):
    """The fp64 oracle on a bounded sample of the workload: the first `sample_rows` batch rows
    x every head over the first `sample_tokens` tokens on every usable host core, then one
    memory over `single_tokens` tokens on one thread.  Rates are workload tokens/s (a token
    is one batch row's position, all heads)."""
    import oracle

    usable = len(os.sched_getaffinity(0))
    T = min(sample_tokens, wl.seq_len)
    rows = min(sample_rows, wl.batch)
    sl = (slice(0, rows), slice(0, T))
    q, k, v = (inp.qkv_f32(n)[sl] for n in ("q", "k", "v"))
    g = [getattr(inp, n)[sl] for n in ("alpha", "eta", "beta")]
    t0 = time.perf_counter()
    oracle.scan(q, k, v, *g, inp.theta0, inp.s0, wl.chunk, wl.widths, nthreads=usable)
    dt = time.perf_counter() - t0
    used = min(usable, rows * wl.heads)
    # one thread, one memory (batch row 0, head 0): memory-tokens/s, / H for workload tokens/s
    T1 = min(single_tokens, wl.seq_len)
    one = (slice(0, 1), slice(0, T1), slice(0, 1))
    q1, k1, v1 = (inp.qkv_f32(n)[one] for n in ("q", "k", "v"))
    g1 = [getattr(inp, n)[one] for n in ("alpha", "eta", "beta")]
    t1 = time.perf_counter()
    oracle.scan(q1, k1, v1, *g1, inp.theta0[:1], inp.s0[:1], wl.chunk, wl.widths, nthreads=1)
    dt1 = time.perf_counter() - t1
    return {"value": rows * T / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "host_cores": os.cpu_count(), "usable_cores": usable,
            "single_thread_value": T1 / dt1 / wl.heads,
            "sample": f"fp64 oracle, batch rows 0..{rows - 1} x all {wl.heads} heads "
                      f"({rows * wl.heads} memories), first {T} of {wl.seq_len} tokens "
                      f"({dt:.1f} s on {used} threads; {usable} usable of {os.cpu_count()} host "
                      f"cores); single thread: 1 memory x {T1} tokens in {dt1:.2f} s"}


def time_calls(torch, fn, steps, warmup):
    """Mean ms of fn() over `steps` calls after `warmup`, from HIP events on torch's current
    stream (the stream the library launches on)."""
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_sustained(tm, torch, t, wl, seed, out, ws, steps, warmup, peak):
    """The same scan (same q, k, v, shapes and launch) with the sustained gate mix, which
    keeps every memory O(1) to the end (with the specified gates the memory decays to its
    zero fixed point within a few thousand tokens, so most chunks of the headline step
    multiply zero state).  Returns the object and the final weights (a live memory)."""
    import synthetic

    swl = synthetic.sustained(wl)
    B, T, H = t["q"].shape[:3]
    gates = synthetic.make_gates(swl, seed, T, B)
    ts = dict(t)
    for n, g in zip(("alpha", "eta", "beta"), gates):
        ts[n] = torch.from_numpy(g).to(t["q"].device)
    y, thT, sT = out

    def run():
        tm.scan(ts["q"], ts["k"], ts["v"], ts["alpha"], ts["eta"], ts["beta"], ts["theta0"],
                ts["s0"], wl.chunk, wl.widths, y=y, theta_T=thT, s_T=sT, workspace=ws)
    ms = time_calls(torch, run, steps, warmup)
    flops = alg_flops_per_token_head(wl.widths, wl.chunk) * B * T * H
    tf = flops / (ms * 1e-3) / 1e12
    fro = thT.double().reshape(B * H, -1).norm(dim=1)
    fin = torch.isfinite(fro)
    # a memory whose weights grow without bound under these gates (the fp64 recurrence
    # diverges on the same draw) is counted, not folded into the norms
    return {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "alpha_mu": swl.alpha_mu,
            "eta_scale": swl.eta_scale, "frac": tf / peak, "achieved": tf,
            "memories_nonfinite": int((~fin).sum()),
            "state_fro_min": float(fro[fin].min()) if fin.any() else None,
            "state_fro_max": float(fro[fin].max()) if fin.any() else None}, thT.clone()


def bench_retrieve(tm, torch, q, theta, wl, steps, warmup):
    """titans_mem_retrieve (fixed-weight read) over the same q with live weights [B, H, P]
    (the sustained scan's final weights, else theta0): its own line, not part of the scan
    step.  Algorithmic bytes: q and y once, theta once per memory; flops 2 P per token-head."""
    y = torch.empty_like(q)
    # the read is short (a fraction of a millisecond at the headline): at least 100 calls,
    # so that clock ramps after the scan's runs average out
    steps = max(steps, 100)
    for _ in range(max(warmup, 5)):
        tm.retrieve(q, theta, wl.widths, y=y)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        tm.retrieve(q, theta, wl.widths, y=y)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    B, T, H, d = q.shape
    io = q.element_size()
    nbytes = 2 * B * T * H * d * io + B * H * wl.params * 4
    flops = 2 * wl.params * B * T * H
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # bound by arithmetic intensity against the bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B):
    # the 64-256-64 read is below it (HBM), wide memories far above it (MFMA)
    if flops / nbytes > PEAKS["mfma_bf16"] * 1e12 / (PEAKS["hbm"] * 1e9) and q.dtype == torch.bfloat16:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAKS["mfma_bf16"], "unit": "TFLOP/s",
                "frac": tflops / PEAKS["mfma_bf16"], "alg_flops_per_launch": flops}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAKS["hbm"], "unit": "GB/s",
                "frac": gbs / PEAKS["hbm"], "alg_bytes_per_launch": nbytes}
    out = {"path": tm.retrieve_path(q, wl.widths), "ms": ms, "calls": steps, "tokens_per_s": B * T / (ms * 1e-3),
           "roofline": roof, "mfma_tflops": tflops}
    # The SiLU of every hidden unit is vector-ALU work: one exp2 and one reciprocal, an add,
    # a multiply and half a packed bf16 conversion.  Priced at the issue costs measured on
    # MI355X relative to an fp32 add (1 slot; exp2 and reciprocal 3.5 each, the packed
    # conversion 1.7) that is 9.85 lane slots per hidden unit and token-head, against
    # 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz = 78.6 T slots/s.  Transcendental VALU work and
    # MFMA work of the waves on one SIMD were measured to overlap little, so the floor of
    # this read is the sum of the two: serial_floor_ms.
    hidden = sum(wl.widths[1:-1])
    if hidden:
        slots = 9.85 * hidden * B * T * H
        rate = slots / (ms * 1e-3) / 1e12
        floor = (slots / (PEAKS["valu_slots"] * 1e12) + flops / (PEAKS["mfma_bf16"] * 1e12)) * 1e3
        out["alu_roofline"] = {"bound": "alu", "achieved": rate, "peak": PEAKS["valu_slots"],
                               "unit": "T lane-slots/s", "frac": rate / PEAKS["valu_slots"],
                               "alg_slots_per_launch": slots, "serial_floor_ms": floor,
                               "serial_frac": floor / ms}
    return out


def bench_biases(tm, torch, t, wl, out, ws, steps, warmup):
    """The same scan with the Huber and l_p attentional biases (their own lines, not part of
    the step): ms per call and tokens/s, to show what the loss derivative costs."""
    y, thT, sT = out
    res = {}
    stream = torch.cuda.current_stream()
    for bias in (("huber", 0.5), ("lp", 3.0)):
        def run():
            tm.scan(t["q"], t["k"], t["v"], t["alpha"], t["eta"], t["beta"], t["theta0"], t["s0"],
                    wl.chunk, wl.widths, y=y, theta_T=thT, s_T=sT, workspace=ws, bias=bias)
        for _ in range(warmup):
            run()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        B, T = t["q"].shape[:2]
        res[f"{bias[0]}_{bias[1]:g}"] = {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
                                         "path": tm.scan_path(t["q"], wl.chunk, wl.widths)}
    return res


def bench_surprise(tm, torch, t, wl, out, steps, warmup):
    """titans_mem_scan_surprise on the same inputs (its own line): the scan plus each
    token's gradient norm, on the generic family (phased for 128+ unit layers)."""
    y, thT, sT = out
    sur = torch.empty_like(t["alpha"])

    def run():  # the binding sizes the workspace for this call's path
        tm.scan(t["q"], t["k"], t["v"], t["alpha"], t["eta"], t["beta"], t["theta0"], t["s0"],
                wl.chunk, wl.widths, y=y, theta_T=thT, s_T=sT, surprise=sur)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    B, T = t["q"].shape[:2]
    return {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "path": tm.surprise_path(t["q"], wl.chunk, wl.widths)}


def bench_backward(tm, torch, t, wl, seed, steps, warmup):
    """titans_mem_scan_backward on the same inputs with seeded output cotangents (its own
    line): tokens/s and the roofline of its two kernels (checkpointing forward sweep,
    reverse chunk loop) against the fp32 matrix-core peak their products run on, timed
    together by HIP events around the call."""
    import synthetic

    cot = synthetic.make_cotangents(wl, seed)
    dev = t["q"].device
    dy = (torch.from_numpy(cot.dy.view(np.int16)).to(dev).view(torch.bfloat16)
          if cot.dy.dtype == np.uint16 else torch.from_numpy(cot.dy).to(dev))
    dth = torch.from_numpy(cot.dtheta_T).to(dev)
    dsT = torch.from_numpy(cot.ds_T).to(dev)
    n = tm.scan_backward_workspace_size(t["q"], wl.chunk, wl.widths)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    out = None

    def run():
        nonlocal out
        out = tm.scan_backward(t["q"], t["k"], t["v"], t["alpha"], t["eta"], t["beta"],
                               t["theta0"], t["s0"], dy, wl.chunk, wl.widths, dtheta_T=dth,
                               ds_T=dsT, workspace=ws, out=out)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    B, T, H = t["q"].shape[:3]
    flops = bwd_alg_flops_per_token_head(wl.widths, wl.chunk) * B * T * H
    tf = flops / (ms * 1e-3) / 1e12
    del ws
    return {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3), "steps": steps,
            "workspace_bytes": n, "kernels": "bwd_forward_kernel + bwd_step_kernel",
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAKS["mfma_f32"],
                         "unit": "TFLOP/s", "frac": tf / PEAKS["mfma_f32"],
                         "alg_flops_per_launch": flops}}


def mag_alg_flops(B, T, H, widths, C, W):
    """Products of one MAG block (memory as gate) by part: the front-end projection
    x W_in^T (2 D (3D + 3H) per token), the memory scan (the scan's own count), causal
    sliding-window attention (4 d per query-key pair: the score dot product and the value
    accumulation; sum_t min(t + 1, W) pairs per (b, h)) and the output projection
    (2 D^2 per token)."""
    d = widths[0]
    D, M = H * d, B * T
    pairs = T * W - W * (W - 1) // 2 if T >= W else T * (T + 1) // 2
    return {"projection": 2.0 * M * D * (3 * D + 3 * H),
            "memory_scan": float(alg_flops_per_token_head(widths, C)) * M * H,
            "attention": 4.0 * d * B * H * pairs,
            "output_projection": 2.0 * M * D * D}


def mac_alg_flops(B, T, H, widths, C, S):
    """Products of one MAC block (memory as context) by part: the front-end projection, the
    memory scan, the memory reads (2 P per token-head), attention (4 d per query-key pair:
    a query of a segment of L tokens sees the L reads and its own causal keys,
    L^2 + L(L+1)/2 pairs per segment and (b, h)) and the output projection."""
    d = widths[0]
    D, M = H * d, B * T
    P = sum(widths[l] * widths[l - 1] for l in range(1, len(widths)))
    pairs = 0
    for t0 in range(0, T, S):
        L = min(S, T - t0)
        pairs += L * L + L * (L + 1) // 2
    return {"projection": 2.0 * M * D * (3 * D + 3 * H),
            "memory_scan": float(alg_flops_per_token_head(widths, C)) * M * H,
            "memory_read": 2.0 * P * M * H,
            "attention": 4.0 * d * B * H * pairs,
            "output_projection": 2.0 * M * D * D}


def bench_mag(tm, torch, wl, window, seed, steps, warmup, kind="mag"):
    """One MAG block (titans_mag_forward; kind="mac": one MAC block, titans_mac_forward,
    with `window` as its segment length) at the workload's shape with model width
    D = H d: x [B, T, D] bf16, seeded weights.  Timed by HIP events around the call on its
    stream; the roofline is the block's algorithmic products against the bf16 matrix-core
    peak (every part runs on bf16 MFMA)."""
    import synthetic

    mi = synthetic.make_mag_inputs(wl, window, seed)
    dev = "cuda"

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w_in, w_out = bf(mi.x), bf(mi.w_in), bf(mi.w_out)
    b_gate = torch.from_numpy(mi.b_gate).to(dev)
    B, H = wl.batch, wl.heads
    th0 = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(mi.theta0, (B,) + mi.theta0.shape))).to(dev)
    s0 = torch.zeros_like(th0)
    size_fn, fwd = ((tm.mag_workspace_size, tm.mag_forward) if kind == "mag"
                    else (tm.mac_workspace_size, tm.mac_forward))
    n = size_fn(x, wl.chunk, window, wl.widths, wl.eta_scale)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    out, thT, sT = torch.empty_like(x), torch.empty_like(th0), torch.empty_like(th0)

    def run():
        fwd(x, w_in, b_gate, w_out, th0, s0, wl.chunk, window, wl.widths, wl.eta_scale,
            out=out, theta_T=thT, s_T=sT, workspace=ws)
    for _ in range(warmup):
        run()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    parts = (mag_alg_flops if kind == "mag" else mac_alg_flops)(B, wl.seq_len, H, wl.widths,
                                                                  wl.chunk, window)
    flops = sum(parts.values())
    tf = flops / (ms * 1e-3) / 1e12
    del ws
    kernels = ("gemm_nt_kernel (projection with the front end) + memory scan + attn_kernel "
               "(sliding window, gated) + gemm_nt_kernel (output)" if kind == "mag" else
               "gemm_nt_kernel (projection with the front end) + per segment: memory read, "
               "memory scan, attn_kernel (read prefix) + gemm_nt_kernel (output)")
    return {"ms": ms, "tokens_per_s": B * wl.seq_len / (ms * 1e-3), "steps": steps,
            "model_width": H * wl.d, ("window" if kind == "mag" else "segment"): window,
            "workspace_bytes": n, "kernels": kernels,
            "alg_flops_by_part": parts,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAKS["mfma_bf16"],
                         "unit": "TFLOP/s", "frac": tf / PEAKS["mfma_bf16"],
                         "alg_flops_per_launch": flops}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-rows", type=int, default=8)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained", action="store_true")
    ap.add_argument("--no-retrieve", action="store_true")
    ap.add_argument("--no-biases", action="store_true")
    ap.add_argument("--no-surprise", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-mag", action="store_true")
    ap.add_argument("--mag-window", type=int, default=4096)
    ap.add_argument("--no-mac", action="store_true")
    ap.add_argument("--mac-segment", type=int, default=4096)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this size first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only: the B*H memories are "
                                   "independent and are not sharded across GPUs; run with --gpus 1"}))
        sys.exit(2)

    import torch

    import sequence_models_amd as tm
    import synthetic

    name = args.workload or synthetic.HEADLINE
    wl = synthetic.WORKLOADS[name]
    inp = synthetic.make_inputs(wl, args.seed)
    dev = torch.device("cuda:0")
    t = {}
    for n in ("q", "k", "v"):
        a = getattr(inp, n)
        t[n] = (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
                if a.dtype == np.uint16 else torch.from_numpy(a).to(dev))
    for n in ("alpha", "eta", "beta", "theta0", "s0"):
        t[n] = torch.from_numpy(getattr(inp, n)).to(dev)
    B, T, H, d = t["q"].shape
    P = wl.params
    y = torch.empty_like(t["q"])
    thT = torch.empty((B, H, P), dtype=torch.float32, device=dev)
    sT = torch.empty_like(thT)
    ws_bytes = tm.scan_workspace_size(t["q"], wl.chunk, wl.widths)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    if args.copy_calibration_mib:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        tm.scan(t["q"], t["k"], t["v"], t["alpha"], t["eta"], t["beta"], t["theta0"], t["s0"],
                wl.chunk, wl.widths, y=y, theta_T=thT, s_T=sT, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ms_per_step = wall * 1e3 / args.steps

    tokens = B * T
    flops = alg_flops_per_token_head(wl.widths, wl.chunk) * B * T * H
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    path = tm.scan_path(t["q"], wl.chunk, wl.widths)
    if path in ("fused_pair", "fused_quad", "fused_mfma"):  # bf16 MFMA, fp32 accumulation
        # the pair path (pairs or quads) is three launches (flag clear, chunk-coefficient
        # pass, scan); the events bracket the whole call, so kernel_ms is their sum
        kernel = ("scan_mfma_kernel" if path == "fused_mfma"
                  else "clear_pair_flags + pair_coef_kernel + scan_pair_kernel")
        bound, peak, dtype = "mfma", PEAKS["mfma_bf16"], "bf16"
    elif path.endswith("_mfma"):  # bf16 MFMA products, fp32 accumulation
        kernel = KERNELS[path.rsplit("_", 1)[0]]
        bound, peak, dtype = "mfma", PEAKS["mfma_bf16"], "bf16"
    elif path.startswith("phased"):  # fp32 FMAs on the vector ALUs
        kernel = KERNELS["phased"]
        bound, peak, dtype = "alu", PEAKS["valu_f32"], "f32"
    else:  # generic / linear fp32: products on the fp32 matrix cores
        kernel = KERNELS[path.rsplit("_", 1)[0]]
        bound, peak, dtype = "mfma", PEAKS["mfma_f32"], "f32"
    parallelism = {
        "fused_pair": "one GPU; two workgroups (one XCD) per (batch row, head) memory",
        "fused_quad": "one GPU; four workgroups (one XCD) per (batch row, head) memory",
        "phased": "one GPU; every chunk product split into 64x64 tiles of all memories, "
                  "4L-2 launches per chunk",
        "linear": "one GPU; each sequence split into groups of chunks whose affine state "
                  "maps compose in parallel",
    }.get(path if path.startswith("fused") else path.split("_")[0],
          "one GPU; one workgroup per (batch row, head) memory")
    result = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": H, "seq_len": T, "d_head": d,
                   "mlp_widths": list(wl.widths), "chunk": wl.chunk, "io": wl.io, "state": "fp32",
                   "parallelism": parallelism, "kernel_path": path},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": measured_traffic(kernel, wl.name),
                     "kernel": kernel, "kernel_ms": kernel_ms,
                     "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes(wl)},
    }
    # fp64 checksums of the final memory per (b, h): its sum and Frobenius norm, listed when
    # there are at most 16 memories (the long-context workload), else summarised
    th64 = thT.double().reshape(B * H, -1)
    sums, fros = th64.sum(dim=1).cpu().tolist(), th64.norm(dim=1).cpu().tolist()
    result["state_checksum"] = ({"sum": sums, "fro": fros} if B * H <= 16 else
                                {"memories": B * H, "sum_total": float(np.sum(sums)),
                                 "fro_min": float(np.min(fros)), "fro_max": float(np.max(fros))})
    import synthetic as _syn
    live = None
    if not args.no_sustained and wl.name in _syn.SUSTAINED:
        result["sustained"], live = bench_sustained(tm, torch, t, wl, args.seed, (y, thT, sT), ws,
                                                    args.steps, args.warmup, peak)
    if not args.no_retrieve:
        if live is None:
            live = t["theta0"].expand(B, -1, -1).contiguous()
        result["retrieve"] = bench_retrieve(tm, torch, t["q"], live, wl, args.steps, args.warmup)
    if not args.no_biases:
        result["biases"] = bench_biases(tm, torch, t, wl, (y, thT, sT), ws, args.steps, args.warmup)
    if not args.no_surprise:
        result["surprise"] = bench_surprise(tm, torch, t, wl, (y, thT, sT), min(args.steps, 5), 1)
    if not args.no_backward:
        result["backward"] = bench_backward(tm, torch, t, wl, args.seed, min(args.steps, 3), 1)
    if not args.no_mag and wl.io == "bf16" and wl.widths[0] == wl.widths[-1]:
        result["mag_block"] = bench_mag(tm, torch, wl, args.mag_window, args.seed,
                                        min(args.steps, 5), 1)
    if not args.no_mac and wl.io == "bf16" and wl.widths[0] == wl.widths[-1]:
        result["mac_block"] = bench_mag(tm, torch, wl, args.mac_segment, args.seed,
                                        min(args.steps, 5), 1, kind="mac")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_sample_rows, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
