"""Benchmark of the KDA forward hot path on one MI355X.

One step = the whole hot path once:
  * kda_chunk_fwd over the K3-shaped prefill (B=1, H=96, T=32768, d=128,
    bf16 q/k/v, fp32 gates and state, state ~ N(0, 0.02)), and
  * one kda_decode_step of the batched decode workload (B=256 sessions, H=96,
    d=128, fp32 state [256, 96, 128, 128] ~ N(0, 0.02)); step s uses token
    s mod 64 of the workload's 64 sequential tokens and updates the state in
    place, so consecutive steps are consecutive decode tokens.

Inputs are seeded synthetic data resident in HBM before timing starts.  Each
kernel is bracketed by HIP events on the stream it runs on (torch's current
stream), so the per-kernel averages are kernel time only.

Output: one JSON line (rank 0).  ``value`` is prefill tokens/s
(B*T / mean kda_chunk_fwd time); the decode figure (state-update GB/s) is in
``decode``; ``ms_per_step`` is the wall time per step (both kernels).
``roofline`` is for kda_chunk_fwd and ``decode.roofline`` for the decode
kernel, both against HBM (8 TB/s).  ``workloads`` times kda_chunk_fwd alone on
the other prefill configurations (tiny fp32, the 4K layer with the Infinity
Cache flushed between repetitions, 16 packed sequences).  ``cpu_baseline`` is
the fp64 oracle on the host cores over all heads of the prefill workload, and
``parity`` compares the timed run's out and final state with it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--no-workloads]       (leave out the other prefill configurations)
       [--copy-calibration]   (adds 1 GiB device copies after timing, used to
                               scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
       [--skip-decode]        (decode workload shrunk to one session-head; for
                               counter passes on kda_chunk_fwd only)
       [--backward [--bwd-workload k3_prefill_32k|prefill_4k|varlen_16]]
                              (instead: kda_chunk_bwd, the gradients of the
                               prefill, on its own JSON line)
       [--prefill-workload tiny|prefill_4k|prefill_4k_f32|varlen_16|k3_prefill_32k|long_1m_h96]
                              (instead: kda_chunk_fwd alone on that workload, dense
                               or packed; its own JSON line)
       [--segments G [--seg-workload long_1m|prefill_4k]]
                              (instead: kda_chunk_fwd_segmented with G requested
                               segments on one long sequence, kda_chunk_fwd
                               timed beside it; its own JSON line)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix, published


def prefill_flop_per_token_head(d=128, C=64):
    """Algorithmic flops per token-head of the chunked prefill, the hot-path
    definition: 6 d_k d_v for the state products ([K+; Q+] S and K_end^T Delta)
    plus C (3 d_k + 2 d_v) + C^2 / 3 for the triangular in-chunk products,
    with d_k = d_v = d and C = 64 (140,629 at d = 128)."""
    return 6 * d * d + C * (3 * d + 2 * d) + C * C / 3


# the kernel's own count (32-token chunks): 6 d^2 plus 24,576 for its
# lower-triangular products (A, Mqk, Delta, Mqk Delta) at d = 128
KERNEL_FLOP_PER_TOKEN_HEAD = 6 * 128 * 128 + 24576
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_fwd_k3_prefill_32k.traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_decode_step_b256.traffic.json")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_chunk_bwd_k3_prefill_32k.traffic.json")
BWD_SOURCES = ("kda_bwd.hip", "kda_bwd_chain.hip", "kda_chunk.hip", "kda_seq.hip", "kda_device.h",
               "kda_lanes.h", "kda_slots.h")
DECODE_SOURCES = ("kda_decode.hip", "kda_device.h")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def prefill_bytes(T_tokens, H, d, n_seqs, esz=2, gate_width=None):
    """Algorithmic HBM bytes of one kda_chunk_fwd: read q, k, v (esz each),
    log_alpha (fp32, gate_width per token-head: d, or 1 for a scalar gate),
    beta (fp32), the initial state; write out (esz) and the final state."""
    gw = d if gate_width is None else gate_width
    per_token_head = 3 * d * esz + 4 * gw + 4 + d * esz
    return T_tokens * H * per_token_head + 2 * n_seqs * H * d * d * 4


def decode_bytes(B, H, d, esz=2, gate_width=None):
    """Algorithmic HBM bytes of one kda_decode_step: the fp32 state read and
    written once, plus q, k, v, log_alpha (gate_width per unit), beta in and out."""
    gw = d if gate_width is None else gate_width
    return B * H * (2 * d * d * 4 + 3 * d * esz + 4 * gw + 4 + d * esz)


def source_digest(names=("kda_chunk.hip", "kda_device.h")):
    """sha256 of a kernel's sources (the prefill's by default) with comments and
    blank lines removed, so that comment edits keep a counter summary valid."""
    import re
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "gated_delta_rule_81_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, names=("kda_chunk.hip", "kda_device.h")):
    """HBM bytes per launch from a committed rocprofv3 counter summary (the
    prefill's by default), if it was taken on the current kernel source; else
    None."""
    try:
        with open(path) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256") != source_digest(names):
        return None
    return doc.get("hbm_bytes_per_launch")


def host_cpu():
    """CPU model name and the cores in this process's affinity mask."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def oracle_threads():
    """Threads for the oracle: every core in the affinity mask, unless
    OMP_NUM_THREADS names the process's share of the host (as it does where
    one host serves several GPUs)."""
    _, cores = host_cpu()
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return min(cores, int(env))
    return cores


def _slice_row_errors(got, ref):
    """Max over heads of the relative L2 error of a [T, h, d] slice, and max
    over token rows of ||x_t - x*_t|| / max(||x*_t||, the slice's RMS row norm)."""
    import numpy as np
    e2 = np.sum((got - ref) ** 2, axis=-1)  # [T, h]
    r2 = np.sum(ref ** 2, axis=-1)
    E, R = e2.sum(axis=0), r2.sum(axis=0)
    slice_err = float(np.max(np.sqrt(E / np.maximum(R, 1e-300))))
    floor = R / max(ref.shape[0], 1)
    row = float(np.max(np.sqrt(e2 / np.maximum(np.maximum(r2, floor), 1e-300))))
    return slice_err, row


def cpu_baseline(inp, heads, threads, out_gpu=None, fin_gpu=None, group=16):
    """The fp64 oracle on `heads` heads of the prefill workload over its full
    length, on the host cores, `group` heads per call; scaled to tokens/s of
    the whole workload.  With the GPU's out / final state of the same
    workload (CPU tensors), also their errors against it on those heads: max
    relative L2 per head slice and per token (state: value) row."""
    import numpy as np
    import oracle

    H = inp["q"].shape[2]
    T = inp["q"].shape[1]
    run = oracle.gdn_forward if inp["log_alpha"].dim() == 3 else oracle.kda_forward
    f = lambda t, h0, h1: t[0, :, h0:h1].float().numpy().astype(np.float64)
    dt = 0.0
    errs = [0.0, 0.0, 0.0, 0.0]  # out slice, out row, state slice, state row
    for h0 in range(0, heads, group):
        h1 = min(heads, h0 + group)
        q, k, v, g = (f(inp[key], h0, h1) for key in ("q", "k", "v", "log_alpha"))
        b = inp["beta"][0, :, h0:h1].numpy().astype(np.float64)
        s0 = inp["initial_state"][:, h0:h1].numpy().astype(np.float64)
        t0 = time.perf_counter()
        ref_out, ref_fin = run(q, k, v, g, b, state0=s0, threads=threads)
        dt += time.perf_counter() - t0
        del q, k, v, g, b
        if out_gpu is not None:
            e = _slice_row_errors(f(out_gpu, h0, h1), ref_out)
            errs[0], errs[1] = max(errs[0], e[0]), max(errs[1], e[1])
            # states: value rows of [h, d_v, d_k] as the token rows of one "slice" per head
            fs = fin_gpu[0, h0:h1].numpy().astype(np.float64).transpose(1, 0, 2)
            e = _slice_row_errors(fs, ref_fin[0].transpose(1, 0, 2))
            errs[2], errs[3] = max(errs[2], e[0]), max(errs[3], e[1])
    model, cores = host_cpu()
    res = {"value": T * heads / dt / H, "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"{heads} of {H} heads x {T} tokens of the prefill workload, "
                     f"fp64, {dt:.1f} s in the oracle; value = sample token-heads/s / {H} "
                     f"heads",
           "cpu_model": model, "affinity_cores": cores}
    parity = None
    if out_gpu is not None:
        parity = {"heads_checked": heads, "of_heads": H, "tokens": T,
                  "out_rel_l2_max": errs[0], "out_row_max": errs[1],
                  "state_rel_l2_max": errs[2], "state_row_max": errs[3],
                  "tol": 2e-2, "row_tol": 4e-2,
                  "metric": "relative L2 per (head) slice, max over slices; rows: "
                            "||x_r - x*_r|| / max(||x*_r||, slice RMS row norm)"}
        parity["pass"] = (errs[0] <= 2e-2 and errs[2] <= 2e-2 and errs[1] <= 4e-2
                          and errs[3] <= 4e-2)
    return res, parity


def attainable_peaks(torch):
    """Measured ceilings to set beside the published ones: HBM bandwidth of a
    4 GiB device-to-device copy (bytes read + written per second) and bf16
    TFLOP/s of an 8192^3 GEMM from the vendor BLAS (calibration only; no part
    of the KDA path uses either)."""
    dev = torch.device("cuda:0")
    n = 1 << 30  # 4 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    y = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(x, y)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2 * m ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    log(f"copy {copy_gbs:.0f} GB/s ({copy_gbs / HBM_PEAK_GBS:.1%} of published); "
        f"bf16 GEMM {tflops:.0f} TFLOP/s ({tflops / BF16_DENSE_PEAK_TFLOPS:.1%} of published)")
    return {"metric": "attainable peaks (calibration)", "hbm_copy_gbs": copy_gbs,
            "hbm_published_gbs": HBM_PEAK_GBS, "bf16_gemm_tflops": tflops,
            "bf16_published_tflops": BF16_DENSE_PEAK_TFLOPS,
            "copy": "4 GiB fp32 device-to-device, read + write bytes",
            "gemm": "torch.matmul bf16 8192 x 8192 x 8192"}


def copy_calibration(torch):
    """Three 1 GiB device-to-device copies after the timed work: their
    rocprofv3 FETCH_SIZE / WRITE_SIZE readings give each counter's scale."""
    dev = torch.device("cuda:0")
    n = 1 << 28  # 1 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copy calibration: 3 x 1 GiB device-to-device copies")


def bwd_bytes(T_tokens, H, d, n_seqs, esz=2):
    """Algorithmic HBM bytes of one kda_chunk_bwd: read q, k, v, d_out (esz),
    log_alpha (fp32), beta, the initial state and the final-state gradient;
    write dq, dk, dv (esz), dlog_alpha (fp32), dbeta and the initial-state
    gradient.  The workspace of chunk states it writes and reads back is
    traffic the method adds, not algorithmic bytes."""
    per_token_head = (4 * d * esz + 4 * d + 4) + (3 * d * esz + 4 * d + 4)
    return T_tokens * H * per_token_head + 3 * n_seqs * H * d * d * 4


# Infinity Cache (MALL) size of the MI355X: workloads smaller than this are
# timed with a write of twice its size between repetitions, outside the timed
# region, so every repetition reads its inputs from HBM.
MALL_BYTES = 256 << 20


def time_prefill(torch, kda, name, steps, warmup, flush=None):
    """kda_chunk_fwd on one named prefill workload (dense or packed; inputs
    seeded and resident in HBM), each repetition timed with HIP events on the
    launch stream.  flush=None: flush the MALL between repetitions when the
    workload's bytes fit in it."""
    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    if w.draw_block:  # too large to draw on the host: drawn on the device, seeded
        log("generating on the device:", w.notes)
        inp = synth.prefill_inputs(w, device=dev)
    else:
        log("generating", w.notes)
        inp = synth.prefill_inputs(w)
    P = {key: inp[key].to(dev) for key in ("q", "k", "v", "log_alpha", "beta")}
    s0 = inp["initial_state"]
    s0 = None if s0 is None else s0.to(dev)
    cu = inp.get("cu_seqlens")
    cu = None if cu is None else cu.to(dev)
    del inp
    B, T, H, D = P["q"].shape
    n_seqs = (cu.numel() - 1) if cu is not None else B
    out = torch.empty_like(P["v"])
    fin = torch.empty((n_seqs, H, D, D), dtype=torch.float32, device=dev)
    tokens = B * T
    esz = P["q"].element_size()
    nbytes = prefill_bytes(tokens, H, D, n_seqs, esz=esz)
    if s0 is None:  # no initial state is read
        nbytes -= n_seqs * H * D * D * 4
    if flush is None:
        flush = nbytes < MALL_BYTES
    scratch = torch.empty(2 * MALL_BYTES // 4, dtype=torch.float32, device=dev) if flush else None
    torch.cuda.synchronize()

    def step():
        kda.chunk_fwd(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], s0, cu, out=out,
                      final_state=fin)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    log(f"timing {steps} x kda_chunk_fwd on {w.name}" + (" (MALL flushed)" if flush else ""))
    t0 = time.perf_counter()
    for s in range(steps):
        if scratch is not None:
            scratch.fill_(float(s))
        ev[s][0].record(stream)
        step()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    avg = sum(ms) / steps
    gbs = nbytes / (avg * 1e-3) / 1e9
    log(f"kda_chunk_fwd on {w.name}: avg {avg:.4f} ms (min {ms[0]:.4f})")
    return {"workload": f"kda_chunk_fwd {w.name}: {w.notes}", "tokens": tokens,
            "sequences": n_seqs, "heads": H, "head_dim": D,
            "dtype": "bf16" if esz == 2 else "f32",
            "tokens_per_s": tokens / (avg * 1e-3), "kernel_ms_avg": avg, "kernel_ms_min": ms[0],
            "kernel_ms_median": ms[steps // 2], "algorithmic_bytes": nbytes,
            "mall_flushed": bool(flush), "wall_s": wall,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None}}


def bench_prefill_workload(torch, args):
    """kda_chunk_fwd alone on one named prefill workload, its own JSON line."""
    import gated_delta_rule_81_amd as kda

    torch.cuda.set_device(torch.device("cuda:0"))
    r = time_prefill(torch, kda, args.prefill_workload, args.steps, args.warmup)
    return {"metric": f"KDA chunked-fwd tokens/s ({args.prefill_workload})",
            "value": r["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": r["wall_s"] / args.steps * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": r["dtype"], "data": "synthetic",
            "config": {"workload": r["workload"], "tokens": r["tokens"],
                       "sequences": r["sequences"], "heads": r["heads"],
                       "head_dim": r["head_dim"], "mall_flushed": r["mall_flushed"]},
            "roofline": r["roofline"], "kernel_ms_avg": r["kernel_ms_avg"],
            "kernel_ms_min": r["kernel_ms_min"], "algorithmic_bytes": r["algorithmic_bytes"],
            "cpu_baseline": None}


def bench_backward(torch, args):
    """kda_chunk_bwd on a prefill workload (inputs and the loss gradients
    seeded, resident in HBM), timed alone with HIP events."""
    import synth
    import gated_delta_rule_81_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.bwd_workload]
    log("generating", w.notes)
    inp = synth.prefill_inputs(w)
    P = {key: inp[key].to(dev) for key in ("q", "k", "v", "log_alpha", "beta")}
    s0 = inp["initial_state"]
    s0 = None if s0 is None else s0.to(dev)
    cu = inp.get("cu_seqlens")
    cu = None if cu is None else cu.to(dev)
    gen = torch.Generator().manual_seed(w.seed + 100)
    Bq, Tq, H, D = P["q"].shape
    T = Bq * Tq
    n_seqs = (cu.numel() - 1) if cu is not None else Bq
    d_out = torch.randn(Bq, Tq, H, D, generator=gen).to(P["q"].dtype).to(dev)
    d_fin = (torch.randn(n_seqs, H, D, D, generator=gen) * 0.1).to(dev)
    ws = torch.empty(kda.bwd_workspace_size(T, n_seqs, H, D), dtype=torch.uint8, device=dev)
    grads = kda.chunk_bwd(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], d_out, d_fin, s0, cu,
                          workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step():
        kda.chunk_bwd(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], d_out, d_fin, s0, cu,
                      workspace=ws, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    log(f"timing {K} x kda_chunk_bwd")
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(K):
        step()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [ev[s].elapsed_time(ev[s + 1]) for s in range(K)]
    avg = sum(ms) / K
    log(f"kda_chunk_bwd: avg {avg:.3f} ms (min {min(ms):.3f})")
    nbytes = bwd_bytes(T, H, D, n_seqs)
    gbs = nbytes / (avg * 1e-3) / 1e9
    # per token-head, in multiply-adds: the forward recompute (K+ S0 and
    # Ke^T Delta: 2 d^2) and the gradient pass (K+ S0, Ke dS, dO S0^T,
    # dX S0^T, Delta dS^T and the state gradient's two products: 7 d^2), plus
    # the 16 x 16 x d products of the 16-token chunks (224 d); flop = 2 x that
    flop = T * H * (18 * D * D + 448 * D)
    tfl = flop / (avg * 1e-3) / 1e12
    # bf16 inputs: bf16 products with fp32 accumulation, so the roofline is the
    # bf16 one, whose ridge (~315 flop/B) lies above this kernel's 125 flop/B
    # of algorithmic intensity: HBM-bound in principle
    bf = P["q"].dtype == torch.bfloat16
    mpeak = BF16_DENSE_PEAK_TFLOPS if bf else FP32_MFMA_PEAK_TFLOPS
    # HBM bytes per call from the committed counter summary (K3 shape only,
    # while the kernel sources are the ones it was taken on)
    traffic = (measured_traffic(BWD_TRAFFIC_FILE, BWD_SOURCES)
               if args.bwd_workload == "k3_prefill_32k" else None)
    if bf:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                "mfma_tflops_algorithmic": tfl, "mfma_frac": tfl / mpeak}
    else:
        roof = {"bound": "mfma", "achieved": tfl, "peak": mpeak, "unit": "TFLOP/s",
                "frac": tfl / mpeak, "traffic": None, "hbm_gbs_algorithmic": gbs,
                "hbm_frac": gbs / HBM_PEAK_GBS}
    return {
        "metric": f"KDA chunked backward tokens/s ({w.notes})",
        "value": T / (avg * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {"workload": f"kda_chunk_bwd {w.name}: {w.notes}; "
                               + ("bf16 products, fp32 accumulation" if bf else "fp32 products")
                               + ", 16-token chunks", "tokens": T, "sequences": n_seqs,
                   "heads": H, "head_dim": D},
        "roofline": roof,
        "kernel_ms_avg": avg, "kernel_ms_min": min(ms), "algorithmic_bytes": nbytes,
        "flop_per_launch": flop,
        "cpu_baseline": None,
    }


def bench_segmented(torch, args):
    """kda_chunk_fwd_segmented on one long sequence (B=1), inputs drawn on the
    device, with kda_chunk_fwd on the same input timed beside it."""
    import synth
    import gated_delta_rule_81_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.seg_workload]
    log("generating on the device:", w.notes)
    P = synth.prefill_inputs(w, device=dev)
    T, H, D = w.seq_len, w.heads, w.head_dim
    G = args.segments
    out = torch.empty_like(P["v"])
    fin = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.segmented_workspace_size(T, H, D, G), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def seg():
        kda.chunk_fwd_segmented(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], G,
                                P["initial_state"], workspace=ws, out=out, final_state=fin)

    def plain():
        kda.chunk_fwd(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], P["initial_state"],
                      out=out, final_state=fin)

    def timed(fn, name, K):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        log(f"timing {K} x {name}")
        ev[0].record(stream)
        for s in range(K):
            fn()
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        ms = [ev[s].elapsed_time(ev[s + 1]) for s in range(K)]
        log(f"{name}: avg {sum(ms) / K:.3f} ms (min {min(ms):.3f})")
        return sum(ms) / K, min(ms)

    t0 = time.perf_counter()
    seg_avg, seg_min = timed(seg, f"kda_chunk_fwd_segmented G={G}", args.steps)
    wall = time.perf_counter() - t0
    plain_avg, plain_min = timed(plain, "kda_chunk_fwd", max(1, min(args.steps, 5)))
    pbytes = prefill_bytes(T, H, D, 1)
    gbs = pbytes / (seg_avg * 1e-3) / 1e9
    seg_tokens = 32 * -(-(-(-T // G)) // 32)  # ceil(T / G) rounded up to whole chunks
    n_seg = -(-T // seg_tokens)
    return {
        "metric": f"KDA segmented prefill tokens/s (B=1 H={H} T={T} d={D})",
        "value": T / (seg_avg * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (wall / args.steps) * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (drawn on the device, seeded)",
        "config": {"workload": f"kda_chunk_fwd_segmented {w.name}: {w.notes}",
                   "requested_segments": G, "segments": n_seg,
                   "segment_tokens": seg_tokens},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "note": "algorithmic bytes of one prefill over the whole segmented "
                             "call (its three passes read the inputs about three times)"},
        "segmented_ms_avg": seg_avg, "segmented_ms_min": seg_min,
        "chunk_fwd_ms_avg": plain_avg, "chunk_fwd_ms_min": plain_min,
        "speedup_vs_chunk_fwd": plain_avg / seg_avg,
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="leave out the timings of the other prefill configurations "
                         "(tiny, prefill_4k, varlen_16) from the default line")
    ap.add_argument("--cpu-heads", type=int, default=96)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--skip-decode", action="store_true",
                    help="time kda_chunk_fwd only (for counter passes); no decode fields")
    ap.add_argument("--attainable", action="store_true",
                    help="measure attainable peaks instead (device-to-device copy for HBM, a "
                         "large bf16 GEMM for the matrix cores) and print them as one JSON line")
    ap.add_argument("--scalar-gate", action="store_true",
                    help="time the scalar-gate (Gated DeltaNet) entry points, one gate per "
                         "token and head (the first channel of the seeded gates)")
    ap.add_argument("--snapshot-every", type=int, default=0,
                    help="time kda_chunk_fwd_snapshots with a state snapshot every N tokens "
                         "(a multiple of 32) instead of kda_chunk_fwd")
    ap.add_argument("--segments", type=int, default=0,
                    help="time kda_chunk_fwd_segmented with this many requested segments "
                         "on one long sequence instead (kda_chunk_fwd timed beside it)")
    ap.add_argument("--seg-workload", default="long_1m", choices=["long_1m", "prefill_4k"],
                    help="the sequence --segments runs on")
    ap.add_argument("--backward", action="store_true",
                    help="time kda_chunk_bwd (the prefill's gradients) instead")
    ap.add_argument("--bwd-workload", default="k3_prefill_32k",
                    choices=["k3_prefill_32k", "prefill_4k", "varlen_16"],
                    help="the prefill workload --backward runs on")
    ap.add_argument("--prefill-workload", default=None,
                    choices=["tiny", "prefill_4k", "prefill_4k_f32", "varlen_16",
                             "k3_prefill_32k", "long_1m_h96"],
                    help="time kda_chunk_fwd alone on this workload instead (its own JSON line)")
    args = ap.parse_args()
    if args.scalar_gate and args.snapshot_every:
        ap.error("--scalar-gate and --snapshot-every time different entry points; pick one")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; multi-GPU runs are not part of it "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.attainable:
        print(json.dumps(attainable_peaks(torch)), flush=True)
        return
    if args.segments > 0:
        print(json.dumps(bench_segmented(torch, args)), flush=True)
        return
    if args.backward:
        res = bench_backward(torch, args)
        if args.copy_calibration:
            copy_calibration(torch)
        print(json.dumps(res), flush=True)
        return
    if args.prefill_workload:
        print(json.dumps(bench_prefill_workload(torch, args)), flush=True)
        return

    import synth
    import gated_delta_rule_81_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w_pre = synth.WORKLOADS["k3_prefill_32k"]
    w_dec = synth.WORKLOADS["decode_b256"]

    log("generating", w_pre.notes)
    pre = synth.prefill_inputs(w_pre)
    if args.skip_decode:
        w_dec = synth.replace(w_dec, batch=1, heads=1, steps=1)
    log("generating", w_dec.notes)
    dec = synth.decode_inputs(w_dec)
    sg = args.scalar_gate
    if sg:  # one gate per (token, head): the first channel of the seeded gates
        pre["log_alpha"] = pre["log_alpha"][..., 0].contiguous()
        dec["log_alpha"] = dec["log_alpha"][..., 0].contiguous()
    P = {key: pre[key].to(dev) for key in ("q", "k", "v", "log_alpha", "beta", "initial_state")}
    Dn = {key: dec[key].to(dev) for key in ("q", "k", "v", "log_alpha", "beta")}
    state = dec["state"].to(dev)
    out = torch.empty_like(P["v"])
    fin = torch.empty_like(P["initial_state"])
    dout = torch.empty((w_dec.batch, w_dec.heads, w_dec.head_dim), dtype=torch.bfloat16,
                       device=dev)
    every = args.snapshot_every
    n_snap = w_pre.batch * (w_pre.seq_len // every) if every > 0 else 0
    snaps = (torch.empty((n_snap, w_pre.heads, w_pre.head_dim, w_pre.head_dim),
                         dtype=torch.float32, device=dev) if every > 0 else None)
    torch.cuda.synchronize()

    def prefill():
        if every > 0:
            kda.chunk_fwd_snapshots(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"], every,
                                    P["initial_state"], out=out, final_state=fin,
                                    snapshots=snaps)
        else:
            kda.chunk_fwd(P["q"], P["k"], P["v"], P["log_alpha"], P["beta"],
                          P["initial_state"], out=out, final_state=fin, scalar_gate=sg)

    def step(s):
        prefill()
        t = s % w_dec.steps
        kda.decode_step(Dn["q"][t], Dn["k"][t], Dn["v"][t], Dn["log_alpha"][t], Dn["beta"][t],
                        state, out=dout, scalar_gate=sg)

    log(f"warmup {args.warmup} steps")
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    stream = torch.cuda.current_stream(dev)
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        t = (args.warmup + s) % w_dec.steps
        kda.decode_step(Dn["q"][t], Dn["k"][t], Dn["v"][t], Dn["log_alpha"][t], Dn["beta"][t],
                        state, out=dout, scalar_gate=sg)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_ms = sorted(ev[s][0].elapsed_time(ev[s][1]) for s in range(K))
    dec_ms = sorted(ev[s][1].elapsed_time(ev[s][2]) for s in range(K))
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K
    log(f"chunk_fwd avg {pre_avg:.4f} ms (min {pre_ms[0]:.4f}, median {pre_ms[K // 2]:.4f}); "
        f"decode_step avg {dec_avg:.4f} ms (min {dec_ms[0]:.4f})")

    if args.copy_calibration:
        copy_calibration(torch)

    T_tok = w_pre.batch * w_pre.seq_len
    gw = 1 if sg else None
    pbytes = prefill_bytes(T_tok, w_pre.heads, w_pre.head_dim, w_pre.batch, gate_width=gw)
    pbytes += n_snap * w_pre.heads * w_pre.head_dim * w_pre.head_dim * 4  # snapshot writes
    dbytes = decode_bytes(w_dec.batch, w_dec.heads, w_dec.head_dim, gate_width=gw)
    pre_gbs = pbytes / (pre_avg * 1e-3) / 1e9
    dec_gbs = dbytes / (dec_avg * 1e-3) / 1e9
    pre_tflops = (prefill_flop_per_token_head(w_pre.head_dim) * T_tok * w_pre.heads
                  / (pre_avg * 1e-3) / 1e12)
    kern_tflops = KERNEL_FLOP_PER_TOKEN_HEAD * T_tok * w_pre.heads / (pre_avg * 1e-3) / 1e12
    traffic = measured_traffic() if every == 0 and not sg else None
    dec_traffic = (measured_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)
                   if not sg and not args.skip_decode else None)

    result = {
        "metric": "KDA chunked-fwd tokens/s (H=96,d=128,T=32K); decode state-update HBM GB/s",
        "value": T_tok / (pre_avg * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("kda_chunk_fwd_scalar_gate" if sg else "kda_chunk_fwd"
                                if every == 0 else
                                f"kda_chunk_fwd_snapshots (every {every} tokens)")
                               + " B=1 H=96 T=32768 d_k=d_v=128 bf16 q/k/v, "
                               "fp32 gates/state, chunk 32 + "
                               + ("kda_decode_step_scalar_gate" if sg else "kda_decode_step")
                               + " B=256 H=96 d=128",
                   "scalar_gate": sg,
                   "snapshot_every": every or None,
                   "prefill_tokens": T_tok, "heads": w_pre.heads, "head_dim": w_pre.head_dim,
                   "decode_sessions": w_dec.batch},
        "roofline": {"bound": "hbm", "achieved": pre_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pre_gbs / HBM_PEAK_GBS,
                     "traffic": traffic},
        "prefill": {"kernel_ms_avg": pre_avg, "kernel_ms_min": pre_ms[0],
                    "kernel_ms_median": pre_ms[K // 2], "algorithmic_bytes": pbytes,
                    "mfma_bf16_tflops_algorithmic": pre_tflops,
                    "mfma_frac_algorithmic": pre_tflops / BF16_DENSE_PEAK_TFLOPS,
                    "mfma_flop_per_token_head": prefill_flop_per_token_head(w_pre.head_dim),
                    "mfma_frac_kernel_count": kern_tflops / BF16_DENSE_PEAK_TFLOPS,
                    "kernel_flop_per_token_head": KERNEL_FLOP_PER_TOKEN_HEAD},
        "decode": {"metric": "decode state-update HBM GB/s", "value": dec_gbs, "unit": "GB/s",
                   "kernel_ms_avg": dec_avg, "kernel_ms_min": dec_ms[0],
                   "algorithmic_bytes": dbytes, "tokens_per_s": w_dec.batch / (dec_avg * 1e-3),
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "traffic": dec_traffic}},
    }
    if not args.no_workloads:
        # the other prefill configurations, each timed alone after the step loop
        result["workloads"] = {}
        for name in ("tiny", "prefill_4k", "varlen_16"):
            result["workloads"][name] = time_prefill(torch, kda, name, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        threads = oracle_threads()
        log(f"cpu baseline: oracle on {args.cpu_heads} heads, {threads} threads; "
            "parity of the timed run's out and final state against it")
        res, parity = cpu_baseline(pre, args.cpu_heads, threads, out.cpu(), fin.cpu())
        result["cpu_baseline"] = res
        result["parity"] = parity
        log(f"parity: {parity}")
    else:
        result["cpu_baseline"] = None
        result["parity"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
