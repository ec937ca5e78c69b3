#!/usr/bin/env python
"""Benchmark of the W4A8 linear layer on one MI355X.

Headline (one JSON line on stdout): decode throughput in GB/s of algorithmic
bytes for one step of the decode workload — per-token int8 quantisation plus
the W4A8 GEMV — at M=1, K=3584 -> N=18944, group 128 (a 7B-decoder MLP
up-projection).  The same line carries:
  roofline      the dominant kernel (the GEMV) against MI355X's 8 TB/s HBM
  cpu_baseline  the CPU oracle timed on this host's cores on the same workload
  prefill       the M=2048 prefill GEMM in int8 TOPS against 5.0 POP/s
  skinny        M=4 and M=16 decode, K=18944 -> N=3584, quant + GEMM
  layer         a 7B-shaped decoder layer's seven linears plus the output
                head, each alone and all from one graph, at M=1 and M=512

Timing: inputs are resident in HBM before the timed region; each timed step
reads a different packed copy of the weights (16 copies, > 512 MB) so the
256 MB Infinity Cache cannot serve them.  Steps run from a captured HIP graph
(the launch-bound inner loop), timed with HIP events on the replay stream; the
dominant kernel's average duration comes the same way from a graph of that
kernel's launches alone (back to back, as rocprofv3 sees them).
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8 linear: decode GB/s (% HBM peak) at M=1; prefill int8 TOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, 2.5 PFLOP/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=256)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--copies", type=int, default=16, help="packed weight copies rotated per step")
    p.add_argument("--prefill-steps", type=int, default=32)
    p.add_argument("--replays", type=int, default=9,
                   help="extra graph replays after the timed one, for the p10/p50/p90 spread")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the skinny and layer legs")
    p.add_argument("--only", choices=["all", "decode", "prefill", "skinny", "layer", "w8a8", "hadamard",
                                      "w4a16", "copy", "peaks"],
                   default="all", help="run one part only (for hardware-counter passes)")
    return p.parse_args()


def measured_traffic(profile):
    """HBM bytes per launch from a committed counter summary under profiles/,
    or None once the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    try:
        kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line and not line.startswith("#"))
        src = open(os.path.join(ROOT, kv["kernel_source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != kv.get("kernel_source_sha256"):
        return None
    return int(kv["traffic_bytes_per_launch"])


def algorithmic_bytes(M, N, K, group=128, act_bytes=2):
    """Bytes the method must move for one linear: packed int4 codes, 4-bit
    zeros, fp32 scales, activations in and bf16 output out."""
    G = K // group
    return N * K // 2 + N * G // 2 + 4 * N * G + act_bytes * M * K + 2 * M * N


def gemm_bytes(M, N, K, group=128):
    """Bytes one GEMM launch must move: packed planes, int8 codes and fp32
    scales of the activations in, bf16 output out."""
    G = K // group
    return N * K // 2 + N * G // 2 + 4 * N * G + M * K + 4 * M + 2 * M * N


def graph_launches_ms(torch, launch, n):
    """Average duration of launch(i) over n back-to-back launches replayed
    from one captured HIP graph (no host gaps between kernels), timed with
    events on the replay stream."""
    return graph_steps_ms(torch, launch, min(n, 8), n) / n


WARM_MS = 30.0  # least device time of untimed replays before a timed one


def graph_steps_ms(torch, step, warmup, steps, spread=None):
    """Capture `steps` calls of step(i) in one HIP graph, replay it, and time
    the replay between a synchronize and events on the replay stream.  The
    untimed warmup replays that same graph max(1, ceil(warmup / steps))
    times first (at least `warmup` steps), and further until WARM_MS of
    replays have run: the first replay of a new graph runs several per cent
    slower than later ones, a one-time cost that a serving loop replaying
    its captured step never pays again, and after the host-side work before
    a measurement (the parity check against the oracle) the first few
    milliseconds of kernels run at a lower clock.  After a synchronize, one
    more untimed replay leads the timed one on the stream, and the events
    bracket only the timed replay: its launch (about 10 us from the replay
    call to the first kernel) overlaps the lead replay, as each step's does
    in a serving loop that replays its captured step back to back, so the
    events time exactly the K steps on the device.  With spread=R the graph
    is replayed R more times after the timed replay, back to back, with an
    event between consecutive replays, and those replay times are kept for
    replay_spread(step, steps)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                 # eager warmup outside capture
        for i in range(min(warmup, 4)):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gt = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gt):
        for i in range(steps):
            step(i)
    t0, n = time.perf_counter(), 0
    while n < max(1, -(-warmup // steps)) or \
            ((time.perf_counter() - t0) * 1e3 < WARM_MS and n < 100000):
        gt.replay()
        torch.cuda.synchronize()
        n += 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gt.replay()                                # untimed lead replay
    e0.record()
    gt.replay()
    e1.record()
    torch.cuda.synchronize()
    first = e0.elapsed_time(e1)
    if spread:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(spread + 1)]
        gt.replay()                            # untimed lead replay
        ev[0].record()
        for r in range(spread):
            gt.replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        _SPREAD[id(step)] = [ev[r].elapsed_time(ev[r + 1]) for r in range(spread)]
    return first


_SPREAD = {}


def replay_spread(step, steps):
    """p10/p50/p90 (microseconds per step) of the extra replays recorded by
    graph_steps_ms(..., spread=R) for this step function."""
    if id(step) not in _SPREAD:
        return None
    t = np.array(_SPREAD.pop(id(step)), dtype=np.float64) * 1e3 / steps
    return {"replays": int(t.size), "steps_per_replay": steps,
            "p10_us": round(float(np.percentile(t, 10)), 3),
            "p50_us": round(float(np.percentile(t, 50)), 3),
            "p90_us": round(float(np.percentile(t, 90)), 3)}


def to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def x_dev(torch, lin):
    x = lin["x"]
    if x.dtype == np.uint16:
        return to_dev(torch, x.view(np.int16)).view(torch.bfloat16)
    return to_dev(torch, x)


def setup_linear(torch, w4, spec, copies):
    from bit_quantized_amd import synth
    lin = synth.make_linear(spec)
    q, z, s = (to_dev(torch, lin[k]) for k in ("q", "z", "s"))
    Ws = [w4.pack_weights(q, z, s) for _ in range(copies)]
    del q, z, s
    x = x_dev(torch, lin)
    return lin, x, Ws


def parity_check(w4, lin, x, W, rows=None, cols=None, windows=None):
    """The benchmarked path against the oracle before timing (on windows of
    rows and columns for the large shapes: `windows` is a list of
    ((m0, m1), (c0, c1)); by default one window of `rows` x `cols`)."""
    import oracle
    y = w4.linear(x, W).float().cpu().numpy()
    qa_ref, sa_ref = oracle.quant_act(lin["x"])
    M, N = lin["spec"].M, lin["spec"].N
    if windows is None:
        windows = [(rows or (0, M), cols or (0, N))]
    worst, out = None, {"windows": []}
    for (m0, m1), (c0, c1) in windows:
        ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(m0, m1),
                            cols=(c0, c1))
        ok, err, bound = oracle.tolerance_ok(y[m0:m1, c0:c1], ref)
        if not ok:
            raise SystemExit(f"parity check failed ({lin['spec'].name}, rows {m0}:{m1}, cols "
                             f"{c0}:{c1}): max err {err:.3e} > {bound:.3e}")
        out["windows"].append({"rows": [m0, m1], "cols": [c0, c1], "max_err": err,
                               "bound": bound})
        if worst is None or err / bound > worst[0] / worst[1]:
            worst = (err, bound)
    out["max_err"], out["bound"] = worst
    if len(windows) == 1:
        w = out.pop("windows")[0]
        out["rows"] = w["rows"]
        if cols:
            out["cols"] = w["cols"]
    return out


def layer_windows(M, N):
    """Parity windows for the layer legs: the first row and (M > 1) a middle
    row from the second row tile and the last row, each over the first and
    the last 64 columns (the last column tiles are the ones a tail split or
    the half tiles take)."""
    rows = [(0, 1)] + ([(M // 2, M // 2 + 1), (M - 1, M)] if M > 1 else [])
    return [(r, c) for r in rows for c in ((0, 64), (N - 64, N))]


def bench_decode(torch, w4, args):
    from bit_quantized_amd import synth
    spec = synth.DECODE_UP
    lin, x, Ws = setup_linear(torch, w4, spec, args.copies)
    M, K, N = spec.M, spec.K, spec.N
    parity = parity_check(w4, lin, x, Ws[0])
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(w4.workspace_bytes(M, N, K), w4.linear_workspace_bytes(M, N, K), 16),
                     dtype=torch.uint8, device="cuda")
    R = len(Ws)

    # the decode step: w4a8_linear = one launch (the GEMV quantises in-kernel)
    def step(i):
        w4.linear(x, Ws[i % R], out=y, workspace=ws)

    total_ms = graph_steps_ms(torch, step, args.warmup, args.steps, spread=args.replays)
    spread = replay_spread(step, args.steps)
    kern_ms = graph_launches_ms(torch, step, args.steps)

    # for reference: the same step as two launches (quantise, then GEMV)
    def two_launch(i):
        w4.quant_act(x, qa, sa)
        w4.gemm(qa, sa, Ws[i % R], out=y, workspace=ws)

    # the floor under the decode step, each from a graph of back-to-back
    # launches like the step itself: a near-empty launch of as many threads
    # as the GEMV (1024 workgroups of 256 threads reading 16 bytes), and the
    # streaming probe reading each packed copy once (the same 36.6 MB per
    # step the GEMV streams, rotated so the Infinity Cache cannot serve it)
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    tiny = torch.zeros(4, dtype=torch.int32, device="cuda")
    empty_ms = graph_launches_ms(torch, lambda i: w4.peak_stream_read(tiny, 1024, sink), args.steps)
    stream = {}
    for blocks in (256, 1024, 2048):
        ms = graph_launches_ms(torch, lambda i, b=blocks: w4.peak_stream_read(Ws[i % R].buf, b, sink),
                               args.steps)
        stream[str(blocks)] = round(ms * 1e3, 3)
    floor = {"empty_launch_us": round(empty_ms * 1e3, 3),
             "stream_packed_copy_us_by_blocks": stream,
             "packed_copy_bytes": int(Ws[0].buf.numel()),
             "gemv_us": round(kern_ms * 1e3, 3),
             "note": "graph-replayed back-to-back launches; a 256-thread workgroup per block"}

    two_ms = graph_steps_ms(torch, two_launch, args.warmup, args.steps) / args.steps
    quant_ms = graph_launches_ms(torch, lambda i: w4.quant_act(x, qa, sa), args.steps)
    gemm_ms = graph_launches_ms(torch, lambda i: w4.gemm(qa, sa, Ws[i % R], out=y, workspace=ws),
                                args.steps)
    step_bytes = algorithmic_bytes(M, N, K)
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = step_bytes / (kern_ms * 1e-3) / 1e9
    path = {1: "gemv", 2: "skinny", 3: "prefill"}[w4.select_path(M, N, K)]
    return {
        "spec": spec, "lin": lin, "value": value, "ms_per_step": ms_per_step,
        "step_bytes": step_bytes, "parity": parity, "path": path, "spread": spread,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("w4a8_gemv_decode_up_M1_K3584_N18944_traffic.txt"),
                     "kernel": f"w4a8 fused quant + {path} (M={M}, K={K}, N={N})",
                     "bytes_per_launch": step_bytes,
                     "avg_launch_us": round(kern_ms * 1e3, 3),
                     "timing": f"{args.steps} launches replayed from one HIP graph (after untimed "
                               "replays of it, the last leading the timed one on the stream)"},
        "floor": floor,
        "two_launch": {"us_per_step": round(two_ms * 1e3, 3),
                       "quant_kernel_us": round(quant_ms * 1e3, 3),
                       "gemv_kernel_us": round(gemm_ms * 1e3, 3),
                       "gemv_GBps": round(gemm_bytes(M, N, K) / (gemm_ms * 1e-3) / 1e9, 1)},
    }


def bench_prefill(torch, w4, args):
    from bit_quantized_amd import synth
    spec = synth.PREFILL_UP
    copies = max(2, min(args.copies, 8))
    lin, x, Ws = setup_linear(torch, w4, spec, copies)
    M, K, N = spec.M, spec.K, spec.N
    parity = parity_check(w4, lin, x, Ws[0], rows=(0, 48))
    qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sa = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    R = len(Ws)

    def step(i):
        w4.quant_act(x, qa, sa)
        w4.gemm(qa, sa, Ws[i % R], out=y)

    n = args.prefill_steps
    total_ms = graph_steps_ms(torch, step, max(2, n // 4), n, spread=args.replays)
    spread = replay_spread(step, n)
    w4.quant_act(x, qa, sa)

    def gemm_only(i):
        w4.gemm(qa, sa, Ws[i % R], out=y)

    kern_ms = graph_steps_ms(torch, gemm_only, min(n, 8), n, spread=args.replays) / n
    kspread = replay_spread(gemm_only, n)
    ops = 2.0 * M * N * K
    tops_kernel = ops / (kern_ms * 1e-3) / 1e12
    tops_step = ops / (total_ms / n * 1e-3) / 1e12
    return {
        "spec": spec, "lin": lin, "parity": parity,
        "workload": f"prefill_up M={M} K={K} N={N} group=128 (quant + GEMM)",
        "value": round(tops_step, 1), "unit": "TOPS", "ms_per_step": total_ms / n,
        "spread": spread, "gemm_spread": kspread,
        "roofline": {"bound": "mfma", "achieved": round(tops_kernel, 1), "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(tops_kernel / INT8_PEAK_TOPS, 4),
                     "traffic": measured_traffic("w4a8_prefill_up_M2048_K3584_N18944_traffic.txt"),
                     "kernel": f"w4a8 prefill (M={M}, K={K}, N={N})",
                     "ops_per_launch": ops, "avg_launch_us": round(kern_ms * 1e3, 2),
                     "timing": f"{n} launches replayed from one HIP graph (after untimed "
                               "replays of it, the last leading the timed one on the stream)"},
    }


def w8_bytes(M, N, K, act_bytes=2):
    """Bytes the W8A8 linear must move: int8 weights, per-channel scales,
    activations in, bf16 output out."""
    return N * K + 4 * N + act_bytes * M * K + 2 * M * N


def bench_w8a8(torch, w4, args):
    """W8A8 int8-dynamic linear: decode (M=1) and skinny (M=4, 16) against the
    HBM roofline, prefill (M=2048) against int8 MFMA peak; each checked
    against the oracle before timing."""
    import oracle
    from bit_quantized_amd import synth
    out = []
    cases = [(synth.LinearSpec("w8_decode_up", 1, 3584, 18944, seed=1), 16),
             (synth.LinearSpec("w8_skinny_down_m4", 4, 18944, 3584, seed=2), 16),
             (synth.LinearSpec("w8_skinny_down_m16", 16, 18944, 3584, seed=2), 16),
             (synth.LinearSpec("w8_prefill_up", 2048, 3584, 18944, seed=3), 4)]
    for spec, copies in cases:
        lin = synth.make_w8_linear(spec)
        qw, sw = to_dev(torch, lin["qw"]), to_dev(torch, lin["sw"])
        Ws = [w4.w8a8_pack_weights(qw, sw) for _ in range(copies)]
        del qw, sw
        x = x_dev(torch, lin)
        M, K, N = spec.M, spec.K, spec.N
        rows = (0, min(M, 16))
        y = w4.w8a8_linear(x, Ws[0])
        qa_ref, sa_ref = oracle.quant_act(lin["x"])
        ref = oracle.w8a8_linear(qa_ref, sa_ref, lin["qw"], lin["sw"], rows=rows)
        ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy()[rows[0]:rows[1]], ref)
        if not ok:
            raise SystemExit(f"parity check failed ({spec.name}): {err:.3e} > {bound:.3e}")
        R = len(Ws)
        ws = torch.empty(max(w4.w8a8_linear_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                         device="cuda")
        n = 64 if M <= 16 else args.prefill_steps
        step_ms = graph_steps_ms(torch, lambda i: w4.w8a8_linear(x, Ws[i % R], out=y, workspace=ws),
                                 max(2, n // 4), n) / n
        qa, sa = w4.quant_act(x)
        gws = torch.empty(max(w4.w8a8_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
        gemm_ms = graph_launches_ms(torch, lambda i: w4.w8a8_gemm(qa, sa, Ws[i % R], out=y,
                                                                  workspace=gws), n)
        r = {"workload": f"{spec.name} M={M} K={K} N={N} (W8A8: quant + int8 GEMM)",
             "path": {1: "gemv", 2: "skinny", 3: "prefill"}[w4.w8a8_select_path(M, N, K)],
             "us_per_step": round(step_ms * 1e3, 3), "gemm_us": round(gemm_ms * 1e3, 3),
             "parity": {"rows": list(rows), "max_err": err, "bound": bound}}
        if M <= 16:
            b = w8_bytes(M, N, K)
            r.update({"bytes_per_step": b, "GBps": round(b / (step_ms * 1e-3) / 1e9, 1),
                      "frac": round(b / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        else:
            ops = 2.0 * M * N * K
            r.update({"ops": ops, "TOPS_step": round(ops / (step_ms * 1e-3) / 1e12, 1),
                      "TOPS_gemm": round(ops / (gemm_ms * 1e-3) / 1e12, 1),
                      "frac_gemm": round(ops / (gemm_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)})
        out.append(r)
        del Ws
    return out


def _rtn_int4(w):
    """Round-to-nearest asymmetric int4 per group of 128 (offline weight
    preparation for the accuracy comparison only): codes, zeros, scales."""
    N, K = w.shape
    g = w.reshape(N, K // 128, 128)
    lo, hi = g.min(axis=2), g.max(axis=2)
    s = np.maximum((hi - lo) / 15.0, 1e-12)
    z = np.clip(np.rint(-lo / s), 0, 15)
    q = np.clip(np.rint(g / s[:, :, None]) + z[:, :, None], 0, 15)
    return (q.reshape(N, K).astype(np.uint8), z.astype(np.uint8), s.astype(np.float32))


def bench_hadamard(torch, w4, args):
    """Online Hadamard rotation + quantisation: its cost against the plain
    quantiser (M = 1, 4, 2048), and what it buys on activations with a few
    large channels: the layer's error against a float64 product, with and
    without the rotation (weights rounded to int4 per group either way, the
    rotated ones from W H / 128)."""
    from bit_quantized_amd import synth
    res = {"timing": []}
    for M, K in ((1, 3584), (4, 18944), (2048, 3584)):
        lin = synth.make_linear(synth.LinearSpec("had", M, K, 16, seed=5), with_weights=False)
        x = x_dev(torch, lin)
        qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        sa = torch.empty((M,), dtype=torch.float32, device="cuda")
        n = 64
        plain = graph_launches_ms(torch, lambda i: w4.quant_act(x, qa, sa), n)
        rot = graph_launches_ms(torch, lambda i: w4.quant_act_hadamard(x, qa, sa), n)
        res["timing"].append({"M": M, "K": K, "quant_us": round(plain * 1e3, 3),
                              "hadamard_quant_us": round(rot * 1e3, 3),
                              "bytes": M * K * 3 + 4 * M})
    # the layer with the rotation against the plain layer: one launch each
    # where the GEMV or the M <= 16 kernel quantises the rows itself
    import oracle
    res["linear"] = []
    for spec in (synth.DECODE_UP, synth.SKINNY_DOWN_4):
        lin, x, Ws = setup_linear(torch, w4, spec, 16)
        M, K, N = spec.M, spec.K, spec.N
        y = w4.linear_hadamard(x, Ws[0])
        qa_ref, sa_ref = oracle.hadamard_quant_act(lin["x"])
        ref = oracle.linear(qa_ref, sa_ref, lin["q"], lin["z"], lin["s"], rows=(0, M))
        ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy(), ref)
        if not ok:
            raise SystemExit(f"parity check failed (hadamard {spec.name}): {err:.3e} > {bound:.3e}")
        R = len(Ws)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(w4.linear_workspace_bytes(M, N, K),
                             int(w4.load().w4a8_linear_hadamard_workspace_bytes(M, N, K, 128)), 16),
                         dtype=torch.uint8, device="cuda")
        plain = graph_launches_ms(torch, lambda i: w4.linear(x, Ws[i % R], out, ws), 64)
        rot = graph_launches_ms(torch, lambda i: w4.linear_hadamard(x, Ws[i % R], out, ws), 64)
        res["linear"].append({"workload": f"{spec.name} M={M} K={K} N={N}",
                              "linear_us": round(plain * 1e3, 3),
                              "linear_hadamard_us": round(rot * 1e3, 3),
                              "parity": {"rows": [0, M], "max_err": err, "bound": bound}})
        del Ws
    # accuracy: 7B-shaped down projection input with 0.5 % of channels x 20
    M, K, N = 16, 3584, 2048
    lin = synth.make_linear(synth.LinearSpec("had_acc", M, K, N, seed=6))
    rng = np.random.Generator(np.random.PCG64(7))
    wf = rng.standard_normal((N, K)) * 0.02
    H = np.array([[(-1) ** bin(a & b).count("1") for b in range(128)] for a in range(128)], np.float64)
    wr = np.concatenate([wf[:, 128 * g:128 * g + 128] @ H / 128.0 for g in range(K // 128)], axis=1)
    xf = synth.x_as_f32(lin).astype(np.float64)
    y_ref = xf @ wf.T
    x = x_dev(torch, lin)
    errs = {}
    for name, wmat, fn in (("plain", wf, w4.linear), ("hadamard", wr, w4.linear_hadamard)):
        q, z, s = _rtn_int4(wmat)
        W = w4.pack_weights(to_dev(torch, q), to_dev(torch, z), to_dev(torch, s))
        y = fn(x, W).float().cpu().numpy().astype(np.float64)
        errs[name] = float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
    res["accuracy"] = {"workload": f"M={M} K={K} N={N}, bf16 N(0,1) activations, 0.5% channels x20, "
                                   "weights N(0, 0.02) rounded to int4 per group",
                       "rel_l2_error_plain": round(errs["plain"], 5),
                       "rel_l2_error_hadamard": round(errs["hadamard"], 5)}
    return res


def bench_w4a16(torch, w4, args):
    """W4A16 (bf16 activations x the packed int4 weights): decode and skinny
    against the HBM roofline, prefill against bf16 MFMA peak; each checked
    against the oracle before timing."""
    import oracle
    from bit_quantized_amd import synth
    out = []
    for spec, copies in ((synth.DECODE_UP, 16), (synth.SKINNY_DOWN_4, 16), (synth.SKINNY_DOWN_16, 16),
                         (synth.PREFILL_UP, 4)):
        lin, x, Ws = setup_linear(torch, w4, spec, copies)
        M, K, N = spec.M, spec.K, spec.N
        rows = (0, min(M, 16))
        y = w4.w4a16_linear(x, Ws[0])
        ref = oracle.w4a16_linear(lin["x"], lin["q"], lin["z"], lin["s"], rows=rows)
        ok, err, bound = oracle.tolerance_ok(y.float().cpu().numpy()[rows[0]:rows[1]], ref)
        if not ok:
            raise SystemExit(f"parity check failed ({spec.name}): {err:.3e} > {bound:.3e}")
        R = len(Ws)
        ws = torch.empty(max(w4.w4a16_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
        n = 64 if M <= 16 else args.prefill_steps
        ms = graph_launches_ms(torch, lambda i: w4.w4a16_linear(x, Ws[i % R], out=y, workspace=ws), n)
        r = {"workload": f"{spec.name} M={M} K={K} N={N} (W4A16: bf16 activations)",
             "path": {1: "gemv", 2: "skinny", 3: "prefill"}[w4.w4a16_select_path(M, N, K)],
             "us": round(ms * 1e3, 3), "parity": {"rows": list(rows), "max_err": err, "bound": bound}}
        if M <= 16:
            b = algorithmic_bytes(M, N, K)
            r.update({"bytes": b, "GBps": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        else:
            flops = 2.0 * M * N * K
            tf = flops / (ms * 1e-3) / 1e12
            r.update({"TFLOPS": round(tf, 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        out.append(r)
        del Ws
    return out


def bench_skinny(torch, w4, args):
    """Skinny decode (2 <= M <= 16): K=18944 -> N=3584 (the configuration
    named for it), then the same batches on the up projection K=3584 ->
    N=18944 (the weight-streaming grid), as quant + GEMM through w4a8_linear,
    against the HBM roofline."""
    from bit_quantized_amd import synth
    out = []
    for spec in (synth.SKINNY_DOWN_4, synth.SKINNY_DOWN_16, synth.SKINNY_UP_4, synth.SKINNY_UP_16):
        lin, x, Ws = setup_linear(torch, w4, spec, args.copies)
        M, K, N = spec.M, spec.K, spec.N
        parity = parity_check(w4, lin, x, Ws[0])
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.zeros(max(w4.linear_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                         device="cuda")
        R = len(Ws)
        n = 64
        step_ms = graph_steps_ms(torch, lambda i: w4.linear(x, Ws[i % R], out=y, workspace=ws),
                                 8, n) / n
        qa = torch.empty((M, K), dtype=torch.int8, device="cuda")
        sa = torch.empty((M,), dtype=torch.float32, device="cuda")
        w4.quant_act(x, qa, sa)
        gws = torch.zeros(max(w4.workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
        gemm_ms = graph_steps_ms(torch, lambda i: w4.gemm(qa, sa, Ws[i % R], out=y, workspace=gws),
                                 8, n) / n
        b = algorithmic_bytes(M, N, K)
        out.append({"workload": f"{spec.name} M={M} K={K} N={N} (quant + GEMM)",
                    "path": {1: "gemv", 2: "skinny", 3: "prefill"}[w4.select_path(M, N, K)],
                    "us_per_step": round(step_ms * 1e3, 3),
                    "GBps": round(b / (step_ms * 1e-3) / 1e9, 1),
                    "frac": round(b / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "gemm_us": round(gemm_ms * 1e3, 3), "bytes_per_step": b, "parity": parity})
        del Ws
    return out


def bench_layer(torch, w4, args):
    """One 7B-shaped decoder layer's linears (q, k, v, o, gate, up, down) and
    the output head, at M=1 (decode) and M=512 (prefill): each linear alone
    (kernel time from a graph of launches), and the eight in sequence from one
    HIP graph (the wall time a layer step would see).  Two packed copies of
    every weight rotate, so the 256 MB Infinity Cache cannot serve them."""
    from bit_quantized_amd import synth
    res = {}
    for M in (1, 512):
        specs = synth.layer_specs(M)
        legs = []
        sib = {}
        for spec in specs:
            lin, x, Ws = setup_linear(torch, w4, spec, 2)
            K, N = spec.K, spec.N
            parity = parity_check(w4, lin, x, Ws[0], windows=layer_windows(M, N))
            y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ws = torch.zeros(max(w4.linear_workspace_bytes(M, N, K), 16), dtype=torch.uint8,
                             device="cuda")
            legs.append({"spec": spec, "x": x, "Ws": Ws, "y": y, "ws": ws, "parity": parity})
            name = spec.name.split("_")[1]
            if name in ("q", "k", "v", "gate", "up"):
                sib[name] = (lin, x)
        rows = []
        for L in legs:
            spec = L["spec"]
            n = 32 if M == 1 else 8
            ms = graph_steps_ms(torch, lambda i, L=L: w4.linear(L["x"], L["Ws"][i % 2], out=L["y"],
                                                               workspace=L["ws"]), 4, n) / n
            r = {"linear": spec.name.split("_")[1], "K": spec.K, "N": spec.N,
                 "us": round(ms * 1e3, 3), "parity_ok": L["parity"]["max_err"] <= L["parity"]["bound"]}
            if M == 1:
                b = algorithmic_bytes(M, spec.N, spec.K)
                r["GBps"] = round(b / (ms * 1e-3) / 1e9, 1)
                r["frac"] = round(r["GBps"] / HBM_PEAK_GBS, 4)
            else:
                ops = 2.0 * M * spec.N * spec.K
                r["TOPS"] = round(ops / (ms * 1e-3) / 1e12, 1)
                r["frac"] = round(r["TOPS"] / INT8_PEAK_TOPS, 4)
            rows.append(r)

        def layer_step(i):
            for L in legs:
                w4.linear(L["x"], L["Ws"][i % 2], out=L["y"], workspace=L["ws"])

        n = 16 if M == 1 else 4
        wall_ms = graph_steps_ms(torch, layer_step, 2, n) / n
        entry = {"linears": rows, "sum_us": round(sum(r["us"] for r in rows), 2),
                 "graph_wall_us": round(wall_ms * 1e3, 2)}

        # sibling projections fused: q/k/v as one weight, gate/up as one (one
        # activation quantisation and one GEMM each); five launches a layer
        fused = []
        for group_names in (("q", "k", "v"), ("gate", "up")):
            parts = [tuple(to_dev(torch, sib[nm][0][k]) for k in ("q", "z", "s"))
                     for nm in group_names]
            Ws = [w4.pack_siblings(parts) for _ in range(2)]
            del parts
            x0 = sib[group_names[0]][1]
            Nf = Ws[0].packed.N
            # parity: every sibling's first and last 64 columns of row 0 and
            # a middle row against the oracle, on the shared input
            import oracle
            lin0 = sib[group_names[0]][0]
            qa_ref, sa_ref = oracle.quant_act(lin0["x"])
            for nm, yv in zip(group_names, w4.linear_siblings(x0, Ws[0])):
                ln = sib[nm][0]
                yn = yv.float().cpu().numpy()
                for (m0, m1), (c0, c1) in layer_windows(M, yn.shape[1]):
                    ref = oracle.linear(qa_ref, sa_ref, ln["q"], ln["z"], ln["s"], rows=(m0, m1),
                                        cols=(c0, c1))
                    ok, err, bound = oracle.tolerance_ok(yn[m0:m1, c0:c1], ref)
                    if not ok:
                        raise SystemExit(f"fused sibling parity failed ({nm}, M={M}, rows "
                                         f"{m0}:{m1}, cols {c0}:{c1})")
            yf = torch.empty((M, Nf), dtype=torch.bfloat16, device="cuda")
            wsf = torch.zeros(max(w4.linear_workspace_bytes(M, Nf, x0.shape[1]), 16),
                              dtype=torch.uint8, device="cuda")
            fused.append({"name": "".join(group_names) if len(group_names) == 3 else "gate_up",
                          "x": x0, "Ws": Ws, "y": yf, "ws": wsf, "N": Nf, "K": x0.shape[1]})
        rest = [L for L in legs if L["spec"].name.split("_")[1] in ("o", "down", "head")]
        frows = []
        for F in fused:
            nn = 32 if M == 1 else 8
            ms = graph_steps_ms(torch, lambda i, F=F: w4.linear(F["x"], F["Ws"][i % 2].packed,
                                                               out=F["y"], workspace=F["ws"]),
                                4, nn) / nn
            frows.append({"linear": F["name"], "K": F["K"], "N": F["N"], "us": round(ms * 1e3, 3)})

        def fused_step(i):
            w4.linear(fused[0]["x"], fused[0]["Ws"][i % 2].packed, out=fused[0]["y"],
                      workspace=fused[0]["ws"])
            L = rest[0]  # o
            w4.linear(L["x"], L["Ws"][i % 2], out=L["y"], workspace=L["ws"])
            w4.linear(fused[1]["x"], fused[1]["Ws"][i % 2].packed, out=fused[1]["y"],
                      workspace=fused[1]["ws"])
            for L in rest[1:]:  # down, head
                w4.linear(L["x"], L["Ws"][i % 2], out=L["y"], workspace=L["ws"])

        fwall_ms = graph_steps_ms(torch, fused_step, 2, n) / n
        entry["fused_siblings"] = {"linears": frows, "graph_wall_us": round(fwall_ms * 1e3, 2)}
        del fused, sib
        if M == 1:
            b = sum(algorithmic_bytes(1, L["spec"].N, L["spec"].K) for L in legs)
            entry["graph_GBps"] = round(b / (wall_ms * 1e-3) / 1e9, 1)
            entry["fused_siblings"]["graph_GBps"] = round(b / (fwall_ms * 1e-3) / 1e9, 1)
        else:
            ops = sum(2.0 * M * L["spec"].N * L["spec"].K for L in legs)
            entry["graph_TOPS"] = round(ops / (wall_ms * 1e-3) / 1e12, 1)
            entry["fused_siblings"]["graph_TOPS"] = round(ops / (fwall_ms * 1e-3) / 1e12, 1)
        res[f"M{M}"] = entry
        del legs
        torch.cuda.empty_cache()
    return res


def cpu_baseline_decode(res, seconds):
    """The oracle as it stands on this host: one decode step = quantise the
    token and compute all N outputs (exact per-group int products, float64
    rescale), repeated for about `seconds`."""
    import oracle
    lin = res["lin"]
    reps, t0 = 0, time.perf_counter()
    while True:
        qa, sa = oracle.quant_act(lin["x"])
        oracle.linear(qa, sa, lin["q"], lin["z"], lin["s"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(res["step_bytes"] * reps / el / 1e9, 3), "unit": "GB/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{reps} full decode steps (quant + all 18944 outputs) in {el:.1f} s"}


def cpu_baseline_prefill(res, seconds):
    import oracle
    lin = res["lin"]
    M, K, N = lin["spec"].M, lin["spec"].K, lin["spec"].N
    t0 = time.perf_counter()
    qa, sa = oracle.quant_act(lin["x"])
    rows, m0 = 0, 0
    while time.perf_counter() - t0 < seconds and m0 < M:
        oracle.linear(qa, sa, lin["q"], lin["z"], lin["s"], rows=(m0, m0 + 8))
        m0 += 8
        rows += 8
    el = time.perf_counter() - t0
    return {"value": round(2.0 * rows * N * K / el / 1e12, 4), "unit": "TOPS",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"quant of all {M} rows + outputs of {rows} rows in {el:.1f} s"}


def cpu_single_thread(runs=10):
    """The oracle on one thread for the tiny, decode and small-batch
    workloads (quantise + every output), median wall time over `runs` calls,
    with the host's CPU model."""
    import oracle
    from bit_quantized_amd import synth
    threads = oracle.threads()
    oracle.set_threads(1)
    out = []
    try:
        for spec in (synth.TINY, synth.DECODE_UP, synth.SKINNY_DOWN_4, synth.SKINNY_DOWN_16):
            lin = synth.make_linear(spec)
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                qa, sa = oracle.quant_act(lin["x"])
                oracle.linear(qa, sa, lin["q"], lin["z"], lin["s"])
                times.append(time.perf_counter() - t0)
            ms = float(np.median(times)) * 1e3
            act = 4 if spec.act == "f32" else 2
            nbytes = algorithmic_bytes(spec.M, spec.N, spec.K, act_bytes=act)
            out.append({"workload": f"{spec.name} M={spec.M} K={spec.K} N={spec.N}",
                        "runs": runs, "median_ms": round(ms, 3),
                        "GBps": round(nbytes / (ms * 1e-3) / 1e9, 3),
                        "GOPS": round(2.0 * spec.M * spec.N * spec.K / (ms * 1e-3) / 1e9, 3)})
    finally:
        oracle.set_threads(threads)
    cpu = _read("/proc/cpuinfo") or ""
    model = next((ln.split(":", 1)[1].strip() for ln in cpu.splitlines()
                  if ln.startswith("model name")), None)
    return {"cores": 1, "kind": "oracle", "cpu_model": model, "timings": out}


def copy_calibration(torch):
    """A plain device copy of known size, for scaling hardware byte counters."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(8):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "launches": 8}))


def bench_peaks(torch, w4):
    """On-device peaks beside the datasheet ones: one read of a 1 GiB buffer
    (four times the 256 MB Infinity Cache) by the streaming probe, and chains
    of v_mfma_i32_16x16x64_i8 on every SIMD with the engine clock they ran
    at (shader cycles over 100 MHz constant-clock ticks)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = 1 << 30
    buf = torch.empty(n // 4, dtype=torch.int32, device="cuda")
    buf.copy_(torch.arange(n // 4, dtype=torch.int32, device="cuda") * 0x01000193)
    res = {"stream_read": [], "mfma_i8": []}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_gbs = 0.0
    for blocks in (4 * cus, 8 * cus, 16 * cus):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        w4.peak_stream_read(buf, blocks, sink)
        times = []
        for _ in range(7):
            e0.record()
            w4.peak_stream_read(buf, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        gbs = [n / (t * 1e-3) / 1e9 for t in times]
        best_gbs = max(best_gbs, float(np.median(gbs)))
        res["stream_read"].append({"blocks": blocks, "bytes": n,
                                   "p10_GBps": round(float(np.percentile(gbs, 10)), 1),
                                   "p50_GBps": round(float(np.median(gbs)), 1),
                                   "p90_GBps": round(float(np.percentile(gbs, 90)), 1)})
    del buf
    best_tops, clk = 0.0, None
    iters = 4096
    for waves_per_simd in (1, 2):
        blocks = cus * waves_per_simd
        sink, clocks = w4.peak_mfma_i8(16, blocks)
        tops, ghz = [], []
        for _ in range(5):
            e0.record()
            w4.peak_mfma_i8(iters, blocks, sink, clocks)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            tops.append(iters * 8 * 32768.0 * blocks * 4 / (ms * 1e-3) / 1e12)
            c = clocks.cpu().numpy().astype(np.float64)
            ghz.append(float(np.median(c[:, 0] / (c[:, 1] / 100e6))) / 1e9)
        med = float(np.median(tops))
        if med > best_tops:
            best_tops, clk = med, float(np.median(ghz))
        res["mfma_i8"].append({"waves_per_simd": waves_per_simd, "blocks": blocks, "iters": iters,
                               "p10_TOPS": round(float(np.percentile(tops, 10)), 1),
                               "p50_TOPS": round(med, 1),
                               "p90_TOPS": round(float(np.percentile(tops, 90)), 1),
                               "sclk_GHz_p50": round(float(np.median(ghz)), 3)})
    res["hbm_GBps"] = round(best_gbs, 1)
    res["int8_TOPS"] = round(best_tops, 1)
    res["sclk_GHz_under_mfma"] = round(clk, 3) if clk else None
    res["note"] = ("on-device peaks measured in this run; the datasheet peaks are 8000 GB/s and "
                   "5000 TOPS (int8 dense, 2.4 GHz)")
    return res


def source_digest():
    """sha256 over the library sources and headers (names and bytes, sorted),
    so a result can be tied to the code it ran."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "bit_quantized_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _read(path):
    try:
        return open(path).read().strip()
    except OSError:
        return None


def dpm_clocks(torch):
    """Current engine (sclk) and memory (mclk) clock levels of this GPU, read
    from the driver's sysfs tables (the starred line of pp_dpm_*), or None."""
    try:
        props = torch.cuda.get_device_properties(0)
        bdf = f"{props.pci_bus_id:02x}:{props.pci_device_id:02x}."
    except Exception:
        return None
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        if bdf not in os.path.basename(os.path.realpath(card)):
            continue
        for clk in ("sclk", "mclk"):
            table = _read(f"{card}/pp_dpm_{clk}") or ""
            cur = [ln.strip() for ln in table.splitlines() if ln.rstrip().endswith("*")]
            if cur:
                out[clk] = cur[0]
        break
    return out or None


def gpu_info(torch):
    info = {"device": torch.cuda.get_device_name(0)}
    try:
        props = torch.cuda.get_device_properties(0)
        info["gcn_arch"] = getattr(props, "gcnArchName", "")
        info["cus"] = props.multi_processor_count
    except Exception:
        pass
    info["source_sha256"] = source_digest()
    info["rocm"] = _read("/opt/rocm/.info/version")
    info["torch"] = torch.__version__
    info["hip"] = getattr(torch.version, "hip", None)
    cpu = _read("/proc/cpuinfo") or ""
    info["cpu_model"] = next((ln.split(":", 1)[1].strip() for ln in cpu.splitlines()
                              if ln.startswith("model name")), None)
    info["host_threads"] = len(os.sched_getaffinity(0))
    import bit_quantized_amd as w4
    lib = w4.load()
    info["abi_version"] = lib.w4a8_abi_version()
    info["layout_version"] = lib.w4a8_layout_version()
    info["w8a8_layout_version"] = lib.w8a8_layout_version()
    info["clocks"] = dpm_clocks(torch)
    info["flags"] = {"env": {k: os.environ[k] for k in ("HIP_VISIBLE_DEVICES", "GPU_MAX_HW_QUEUES",
                                                         "OMP_NUM_THREADS") if k in os.environ}}
    return info


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the W4A8 linear here has no multi-GPU path "
              "(sharding is a design note only); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_amd as w4
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w4.load()
    if args.only == "copy":
        copy_calibration(torch)
        return

    dec = pre = skinny = layer = w8 = had = a16 = peaks = None
    if args.only in ("all", "decode"):
        dec = bench_decode(torch, w4, args)
    if args.only in ("all", "prefill") and not args.no_prefill:
        pre = bench_prefill(torch, w4, args)
    if args.only == "skinny" or (args.only == "all" and not args.no_extra):
        skinny = bench_skinny(torch, w4, args)
    if args.only == "layer" or (args.only == "all" and not args.no_extra):
        layer = bench_layer(torch, w4, args)
    if args.only == "w8a8" or (args.only == "all" and not args.no_extra):
        w8 = bench_w8a8(torch, w4, args)
    if args.only == "hadamard" or (args.only == "all" and not args.no_extra):
        had = bench_hadamard(torch, w4, args)
    if args.only == "w4a16" or (args.only == "all" and not args.no_extra):
        a16 = bench_w4a16(torch, w4, args)
    # the peak probes last: their int8 MFMA chains run the matrix cores at
    # full power, and the memory-bound decode step measured about 3 % slower
    # right after them
    if args.only in ("all", "peaks"):
        peaks = bench_peaks(torch, w4)
    cpu_dec = cpu_pre = None
    if not args.no_cpu_baseline and args.only == "all":
        if dec:
            cpu_dec = cpu_baseline_decode(dec, args.cpu_seconds)
        if pre:
            cpu_pre = cpu_baseline_prefill(pre, max(2.0, args.cpu_seconds / 3))
        if cpu_dec:
            cpu_dec["single_thread"] = cpu_single_thread()

    from bit_quantized_amd import synth
    if peaks:
        # the same kernels against what this device reached in this run
        for leg, key in ((dec, "hbm_GBps"), (pre, "int8_TOPS")):
            if leg and peaks.get(key):
                rf = leg["roofline"]
                rf["peak_onbox"] = peaks[key]
                rf["frac_onbox"] = round(rf["achieved"] / peaks[key], 4)
    if dec is None:
        out = {"metric": METRIC}
        if peaks:
            out["peaks"] = peaks
        if pre:
            out["prefill"] = {k: v for k, v in pre.items() if k not in ("spec", "lin")}
        if skinny:
            out["skinny"] = skinny
        if layer:
            out["layer"] = layer
        if w8:
            out["w8a8"] = w8
        if had:
            out["hadamard"] = had
        if a16:
            out["w4a16"] = a16
        print(json.dumps(out))
        return
    spec = dec["spec"]
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"decode_up M={spec.M} K={spec.K} N={spec.N} group=128 "
                               f"(per-token int8 quant fused into the W4A8 {dec['path']})",
                   "M": spec.M, "K": spec.K, "N": spec.N, "group": 128,
                   "activations": "bf16 N(0,1), 0.5% channels x20", "seed": spec.seed,
                   "input_sha256_16": synth.digest(dec["lin"]), "weight_copies": args.copies,
                   "bytes_per_step": dec["step_bytes"],
                   "timing": "one timed replay of a HIP graph of K steps, after max(1, ceil(W / K)) "
                             "untimed replays of the same graph and at least %g ms of them; after "
                             "a synchronize one untimed replay leads the timed one on the stream "
                             "and events bracket the timed replay alone" % WARM_MS,
                   "parallelism": "single GPU"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu_dec,
        "two_launch": dec["two_launch"],
        "decode_floor": dec["floor"],
        "parity": dec["parity"],
    }
    if dec.get("spread"):
        line["spread"] = dec["spread"]
    if peaks:
        line["peaks"] = peaks
    if pre:
        p = {k: v for k, v in pre.items() if k not in ("spec", "lin")}
        p["cpu_baseline"] = cpu_pre
        line["prefill"] = p
    if skinny:
        line["skinny"] = skinny
    if layer:
        line["layer"] = layer
    if w8:
        line["w8a8"] = w8
    if had:
        line["hadamard"] = had
    if a16:
        line["w4a16"] = a16
    line["system"] = gpu_info(torch)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
