#!/usr/bin/env python3
"""Throughput of the looped W4A4 group-quantized linear on one MI355X.

One step = one looped forward of an Ouro-1.4B-like block over T loops: for
each quantized input (qkv_in feeding the fused q/k/v weight, o_in, up_in,
down_in) the fused Kronecker transform + group RTN quantizer and the integer
GEMM with per-group rescale, with the same packed INT4 weights at every loop
and one LAS clip per input and loop.  Inputs (bf16 activations, packed
weights, factors) are resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Prints one JSON line.  ``value`` is algorithmic GEMM ops (2*M*N*K summed over
the step's linears and loops) per second of wall time, in TOPS.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "looped W4A4 linear TOPS & GB/s per loop-step, % of INT8-MFMA/HBM roofline"
INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--M", type=int, default=1024)
    p.add_argument("--T", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="rows in the oracle sample (0 = auto)")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many steps of the W4A4 step (for rocprofv3), no JSON")
    p.add_argument("--profile-schedule", type=int, default=0,
                   help="schedule used by --profile-steps (0 auto, 1 loop-sequential, 2 weight-stationary)")
    p.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    p.add_argument("--no-loop-dependent", action="store_true",
                   help="skip the loop-dependent (per-loop weight sets / bit widths) measurement")
    p.add_argument("--no-hessian", action="store_true", help="skip the trajectory Hessian measurement")
    p.add_argument("--no-recurrence", action="store_true", help="skip the adapter recurrence measurement")
    p.add_argument("--no-per-token", action="store_true", help="skip the per-token measurement")
    p.add_argument("--profile-hessian", type=int, default=0,
                   help="only run this many trajectory Hessian steps (for a profiler) and exit")
    p.add_argument("--decode-steps", type=int, default=20)
    p.add_argument("--profile-decode", type=int, default=0,
                   help="only run this many decode loop-steps at M=1 (for rocprofv3), no JSON")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="with --profile-steps: first run one device-to-device copy of this many MiB "
                        "(a plain copy kernel of known size that calibrates HBM byte counters)")
    return p.parse_args()


class Module:
    """One quantized input and the (fused) weight that reads it."""

    def __init__(self, act, K, N, P1, P2, clips, x, codes, scales):
        self.act, self.K, self.N = act, K, N
        self.P1, self.P2, self.clips = P1, P2, clips
        self.x, self.codes, self.scales = x, codes, scales
        self.y = None
        self.ws = None


def build_modules(lq, synth, wl, torch):
    """Group the block's linears by quantized input (q, k, v share qkv_in and
    are packed as one weight of N = 3 * hidden), draw inputs, pack weights."""
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.act, []).append(lin)
    mods = []
    for act, lins in groups.items():
        K = lins[0].K
        W = __import__("numpy").concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        N = W.shape[0]
        codes, scales = lq.empty_packed_weights(K, N, wl.group_w)
        lq.loopq_pack_weights(torch.from_numpy(W).cuda(), wl.group_w, codes, scales)
        P1, P2 = synth.factors_for(wl, act, K)
        bits, _ = synth.activations_for(wl, act, K)
        x = torch.from_numpy(bits.view(__import__("numpy").int16)).cuda().view(torch.bfloat16)
        mods.append(Module(act, K, N, torch.from_numpy(P1).cuda(), torch.from_numpy(P2).cuda(),
                           [float(c) for c in synth.clips_for(wl, act)], x, codes, scales))
    return mods


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "hbm_traffic_ouro_block_M1024_T4.md")


def gemm_source_sha256():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in ("bit_ptq_looped_amd/csrc/gemm_f6.hip", "bit_ptq_looped_amd/csrc/gemm_tile.h"):
        with open(os.path.join(root, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per GEMM launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the GEMM source changed since it was taken."""
    try:
        fields = dict(line.split(": ", 1) for line in open(TRAFFIC_FILE).read().splitlines()
                      if line.startswith("gemm_"))
    except OSError:
        return None
    if fields.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    return float(fields["gemm_traffic_bytes_per_launch"])


HESSIAN_TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                    "hbm_traffic_trajectory_hessian_ouro_block_M1024_T4.md")


def hessian_traffic():
    """Counter bytes per trajectory Hessian step from the committed summary,
    or None when hessian.hip changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        fields = dict(line.split(": ", 1) for line in open(HESSIAN_TRAFFIC_FILE).read().splitlines()
                      if line.startswith("hessian_"))
        with open(os.path.join(root, "bit_ptq_looped_amd/csrc/hessian.hip"), "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
    except OSError:
        return None
    if fields.get("hessian_source_sha256") != sha:
        return None
    return float(fields["hessian_traffic_bytes_per_step"])


VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9  # fp32 lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz


def fold_inclusive(mods, T, M, gemm_ms):
    """The GEMM against a bound that counts the per-group fold: M*N*K/32
    element-groups per loop, each an fp32 product of the two steps and an FMA
    into the accumulator (2 VALU lane operations, no packed math), plus the
    MFMA time of the integer ops.  On gfx950 MFMA and VALU issue cycles add,
    so the bound is the sum."""
    groups = sum(T * M * m.N * m.K / 32.0 for m in mods)
    t_fold = 2.0 * groups / VALU_LANE_OPS
    t_mfma = alg_ops(mods, T, M) / (INT8_PEAK_TOPS * 1e12)
    return {"element_groups_per_step": groups, "t_fold_ms": t_fold * 1e3, "t_mfma_ms": t_mfma * 1e3,
            "bound_ms": (t_fold + t_mfma) * 1e3, "gemm_ms": gemm_ms,
            "frac": (t_fold + t_mfma) * 1e3 / gemm_ms}


def alg_ops(mods, T, M):
    return sum(2.0 * T * M * m.N * m.K for m in mods)


def alg_bytes_per_loop_step(mods, M, group_w):
    """Packed weights + fp16 steps + bf16 activations in + fp32 y out, once per loop-step."""
    b = 0.0
    for m in mods:
        b += m.N * m.K / 2 + 2 * m.N * (m.K // group_w)
        b += 2 * M * m.K + 4 * M * m.N
    return b


def run_steps(lq, mods, bits, schedule, steps):
    for _ in range(steps):
        for m in mods:
            lq.loopq_looped_forward(m.x, m.P1, m.P2, m.clips, bits, m.codes, m.scales, 32, m.N, m.y,
                                    schedule, m.ws)


def timed(lq, torch, mods, bits, schedule, steps, warmup, hooks=False):
    run_steps(lq, mods, bits, schedule, warmup)
    torch.cuda.synchronize()
    lq.loopq_timing_reset()
    if hooks:
        lq.loopq_timing_enable(True)
    t0 = time.perf_counter()
    run_steps(lq, mods, bits, schedule, steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lq.loopq_timing_enable(False)
    per_kernel = lq.loopq_timing_read(3)
    return (t1 - t0) / steps, per_kernel


DECODE_LAYERS = 24


def build_decode(lq, synth, torch, M, T, layers=DECODE_LAYERS):
    """The Ouro-like block at decode size: per quantized input, one loop's
    M rows (bf16), the input's factors and clips, and packed weights for
    `layers` distinct layers.  Layer 0 packs the seeded weights; deeper layers
    get seeded random packed bytes and fp16 steps drawn on the device (kernel
    time does not depend on the values; parity runs on layer 0 shapes)."""
    import numpy as np
    wl = synth.ouro_block_workload(bits_a=4, M=M, T=T)
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.act, []).append(lin)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260)
    mods = []
    for act, lins in groups.items():
        K = lins[0].K
        W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        N = W.shape[0]
        P1, P2 = synth.factors_for(wl, act, K)
        bits, _ = synth.activations_for(wl, act, K)
        x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)  # [T][M][K]
        weights = []
        for layer in range(layers):
            codes, scales = lq.empty_packed_weights(K, N, wl.group_w)
            if layer == 0:
                lq.loopq_pack_weights(torch.from_numpy(W).cuda(), wl.group_w, codes, scales)
            else:
                codes.copy_(torch.randint(0, 256, codes.shape, dtype=torch.uint8, device="cuda", generator=gen))
                steps = (torch.rand(scales.numel() // 2, device="cuda", generator=gen) * 0.01 + 0.001)
                scales.copy_(steps.to(torch.float16).view(torch.uint8))
            weights.append((codes, scales))
        m = Module(act, K, N, torch.from_numpy(P1).cuda(), torch.from_numpy(P2).cuda(),
                   [float(c) for c in synth.clips_for(wl, act)], x, None, None)
        m.weights = weights
        m.y1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        m.yT = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
        m.ws1 = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, 1, M, K, N, 4)
        m.wsT = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4)
        mods.append(m)
    return wl, mods


def decode_loop_step(lq, mods, t):
    """One loop-step of the decode stack: every layer's quantized inputs
    (loop t's rows, loop t's clips) through that layer's weights."""
    for layer in range(DECODE_LAYERS):
        for m in mods:
            codes, scales = m.weights[layer]
            lq.loopq_looped_forward(m.x[t:t + 1], m.P1, m.P2, [m.clips[t]], 4, codes, scales, 32, m.N,
                                    m.y1, lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.ws1)


def decode_bench(lq, synth, torch, M, T, steps):
    wl, mods = build_decode(lq, synth, torch, M, T)
    per_layer_bytes = sum(m.N * m.K / 2 + 2 * m.N * (m.K // 32) for m in mods)
    act_bytes = sum(2 * M * m.K + 4 * M * m.N for m in mods)
    step_bytes = DECODE_LAYERS * (per_layer_bytes + act_bytes)
    for t in range(2):
        decode_loop_step(lq, mods, t % T)
    torch.cuda.synchronize()
    lq.loopq_timing_reset()
    lq.loopq_timing_enable(True)
    for i in range(steps):
        decode_loop_step(lq, mods, i % T)
    torch.cuda.synchronize()
    lq.loopq_timing_enable(False)
    kern = lq.loopq_timing_read(4)
    launches = sum(n for _, n in kern) / steps
    t0 = time.perf_counter()
    for i in range(steps):
        decode_loop_step(lq, mods, i % T)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    fused_ms = kern[lq.LOOPQ_KERNEL_DECODE][0] / steps  # the few-row kernel (one launch per call where it can)
    # the same loop-steps replayed from a captured graph (launch gaps only):
    # loops 0..T-1 once each per replay; outputs checked against eager runs
    eager_ref = []
    for t in range(T):
        decode_loop_step(lq, mods, t)
    torch.cuda.synchronize()
    eager_ref = [m.y1.clone() for m in mods]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for t in range(T):
                decode_loop_step(lq, mods, t)
    torch.cuda.current_stream().wait_stream(cap)
    graph_ok = True
    for _ in range(3):
        for m in mods:
            m.y1.zero_()
        graph.replay()
        torch.cuda.synchronize()
        graph_ok &= all(torch.equal(m.y1, r) for m, r in zip(mods, eager_ref))
        decode_loop_step(lq, mods, 0)  # eager work between replays
        torch.cuda.synchronize()
    reps_g = max(1, steps // T)
    t0 = time.perf_counter()
    for _ in range(reps_g):
        graph.replay()
    torch.cuda.synchronize()
    graph_wall = (time.perf_counter() - t0) / (reps_g * T)
    del graph
    # reuse run: layer 0 looped T times in one weight-stationary call per input
    for m in mods:
        codes, scales = m.weights[0]
        lq.loopq_looped_forward(m.x, m.P1, m.P2, m.clips, 4, codes, scales, 32, m.N, m.yT,
                                lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.wsT)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 50
    for _ in range(reps):
        for m in mods:
            codes, scales = m.weights[0]
            lq.loopq_looped_forward(m.x, m.P1, m.P2, m.clips, 4, codes, scales, 32, m.N, m.yT,
                                    lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.wsT)
    torch.cuda.synchronize()
    reuse = (time.perf_counter() - t0) / reps
    return {
        "M": M, "layers": DECODE_LAYERS, "loops": T,
        "ms_per_loop_step": wall * 1e3,
        "gbps_per_loop_step": step_bytes / wall / 1e9,
        "frac_hbm_peak": step_bytes / wall / 1e9 / HBM_PEAK_GBS,
        "kernel_ms_per_loop_step": {"decode": fused_ms,
                                    "transform_items_and_quantizer": sum(kern[k][0] for k in (
                                        lq.LOOPQ_KERNEL_QUANT_TRANSFORM, lq.LOOPQ_KERNEL_QUANT_PLAIN)) / steps},
        "launches_per_loop_step": launches,
        "bytes_per_loop_step": step_bytes,
        "graph_ms_per_loop_step": graph_wall * 1e3,
        "graph_gbps_per_loop_step": step_bytes / graph_wall / 1e9,
        "graph_frac_hbm_peak": step_bytes / graph_wall / 1e9 / HBM_PEAK_GBS,
        "graph_replays_match_eager": bool(graph_ok),
        "reuse_one_layer_T_loops_ms": reuse * 1e3,
        "reuse_weight_bytes_per_loop": per_layer_bytes / T,
    }


def loop_dependent_bench(lq, synth, torch, wl, mods, steps, warmup):
    """The block with loop-dependent pieces (loopq_looped_forward_ex): every
    loop with its own packed weights and factors (SLT selecting every module:
    no weight sharing), and a per-loop activation width table (A8 for loop 0,
    A4 after) on the shared weights.  Same step, inputs and algorithmic ops."""
    import numpy as np
    T, M = wl.T, wl.M
    for m in mods:
        own = []
        for t in range(T):
            W = np.concatenate([synth.weights_for(wl, lin, layer=1 + t) for lin in
                                [l for l in wl.linears if l.act == m.act]], axis=0)
            codes, scales = lq.empty_packed_weights(m.K, m.N, wl.group_w)
            lq.loopq_pack_weights(torch.from_numpy(W).cuda(), wl.group_w, codes, scales)
            own.append((codes, scales))
        m.own_weights = own
        m.own_factors = [(m.P1, m.P2)] + [tuple(torch.from_numpy(f).cuda() for f in
                                                synth.factors_for(wl, m.act, m.K, layer=1 + t)) for t in range(1, T)]
        m.ws_ex = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_EX, T, M, m.K, m.N, 0)

    def run(kind, n):
        for _ in range(n):
            for m in mods:
                if kind == "slt":
                    lq.loopq_looped_forward_ex(m.x, m.own_factors, m.clips, [4] * T, m.own_weights, 32, m.N,
                                               m.y, list(range(T)), m.ws_ex)
                else:
                    lq.loopq_looped_forward_ex(m.x, [(m.P1, m.P2)], m.clips, [8] + [4] * (T - 1),
                                               [(m.codes, m.scales)], 32, m.N, m.y, [0] * T, m.ws_ex)

    out = {}
    ops = alg_ops(mods, T, M)
    for kind in ("slt", "bits_8444"):
        run(kind, warmup)
        dt, blocks = median_blocks(torch, lambda n: run(kind, n), steps)
        out[kind] = {"ms_per_step": dt * 1e3, "value": ops / dt / 1e12, "blocks_ms_per_step": blocks}
    out["slt"]["what"] = ("every loop with its own packed weights and factors (no sharing): per input, one "
                          "quantizer launch per loop and one grouped GEMM over all T*M rows")
    out["bits_8444"]["what"] = "loop 0 at A8, loops 1-3 at A4, shared weights: two weight-stationary runs per input"
    return out


def median_blocks(torch, run, steps, blocks=3):
    """Wall time per step of run(steps), taken as `blocks` separately timed
    blocks: (median seconds per step, each block's ms per step).  The
    secondary lines have read 3-4x their usual time in single runs now and
    then, for a cause not established; the median keeps one such block from
    setting the figure, and the block list shows it."""
    per = []
    for _ in range(blocks):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        per.append((time.perf_counter() - t0) / steps)
    return sorted(per)[len(per) // 2], [round(p * 1e3, 4) for p in per]


def per_token_bench(lq, torch, mods, T, M, steps, warmup):
    """The block's step with one activation step per token (the
    rtn_w4a4_per_token arm) on the same transforms and packed weights: per
    quantized input one loopq_looped_forward_per_token over all T loops
    (transform kernel with per-row steps, one weight-stationary GEMM).  Same
    algorithmic ops."""
    for m in mods:
        m.ws_tok = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, m.K, m.N, 4)

    def run(n):
        for _ in range(n):
            for m in mods:
                lq.loopq_looped_forward_per_token(m.x, m.P1, m.P2, m.clips, 4, m.codes, m.scales, 32, m.N, m.y,
                                                  m.ws_tok)

    run(warmup)
    dt, blocks = median_blocks(torch, run, steps)
    for m in mods:
        del m.ws_tok
    return {"what": "per-token activation steps, W4A4, all T loops of an input in one weight-stationary call",
            "ms_per_step": dt * 1e3, "value": alg_ops(mods, T, M) / dt / 1e12, "unit": "TOPS",
            "blocks_ms_per_step": blocks}


def recurrence_bench(lq, synth, torch, M, T, steps):
    """The Huginn-like adapter loop (adapter 10560 -> 5280, weight groups of
    128, A8, no transform): T dependent loops s_{t+1} = adapter(cat(s_t, e))
    in one loopq_recurrent_adapter call.  The weight is drawn N(0, (0.5 /
    sqrt(K))^2) so the state keeps its scale over 32 loops (timing does not
    depend on the values).  Per loop: 2 M N K ops; bytes = packed weight and
    steps + the fp32 x read + the fp32 y written."""
    import numpy as np
    N, K, gw, bits = 5280, 10560, 128, 8
    rng = synth.seeded_rng(synth.HUGINN, synth.T_W, 99)
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.5 / np.sqrt(K)))
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(torch.from_numpy(w).cuda(), gw, codes, scales)
    del w
    s0 = torch.from_numpy(synth.seeded_rng(synth.HUGINN, synth.T_X, 99).standard_normal((M, N), dtype=np.float32)).cuda()
    e = torch.from_numpy(synth.seeded_rng(synth.HUGINN, synth.T_AUX, 99).standard_normal((M, N), dtype=np.float32)).cuda()
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, M, 0, N, bits), dtype=torch.uint8,
                     device="cuda")
    clips = [1.0] * T
    lq.loopq_recurrent_adapter(s0, e, None, None, clips, bits, codes, scales, gw, y, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lq.loopq_recurrent_adapter(s0, e, None, None, clips, bits, codes, scales, gw, y, ws)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps / T
    wbytes = codes.numel() + scales.numel()
    loop_bytes = wbytes + 4.0 * M * K + 4.0 * M * N
    finite = bool(torch.isfinite(y).all().item())
    return {"M": M, "T": T, "N": N, "K": K, "group_w": gw, "bits": "W4A8", "ms_per_loop": dt * 1e3,
            "tops": 2.0 * M * N * K / dt / 1e12, "gbps": loop_bytes / dt / 1e9,
            "frac_hbm_peak": loop_bytes / dt / 1e9 / HBM_PEAK_GBS, "weight_bytes": wbytes,
            "states_finite": finite}


def hessian_setup(lq, torch, mods, T, M):
    """x~ of every loop of each quantized input (the quantizer's dump, formed
    once, untimed), a zeroed fp32 [K][K] Hessian and the workspace per input."""
    for m in mods:
        rows = T * M
        x2 = m.x.reshape(rows, m.K)
        codes = torch.empty((rows, m.K), dtype=torch.int8, device="cuda")
        steps = torch.empty((rows, m.K // 32), dtype=torch.float32, device="cuda")
        m.xt = torch.empty((rows, m.K), dtype=torch.float32, device="cuda")
        lq.loopq_quant_act(x2, m.P1, m.P2, 1.0, 4, codes, steps, m.xt)
        m.H = torch.zeros((m.K, m.K), dtype=torch.float32, device="cuda")
        m.ws_h = lq.empty_workspace(lq.LOOPQ_OP_HESSIAN, 0, rows, m.K, 0, 0)
        del codes, steps
    torch.cuda.synchronize()


def hessian_step(lq, mods):
    for m in mods:
        lq.loopq_hessian_accumulate(m.xt, m.H, m.ws_h)


def hessian_bench(lq, torch, mods, T, M, steps, warmup):
    """Trajectory Hessian H += x~^T x~ over the x~ rows of all T loops, one
    accumulation per quantized input of the block (K = 2048 three times,
    K = 5632 once).  Algorithmic flops: rows * K * (K + 1) per input (the
    multiply-adds of the upper triangle with the diagonal)."""
    hessian_setup(lq, torch, mods, T, M)
    for _ in range(warmup):
        hessian_step(lq, mods)
    torch.cuda.synchronize()
    lq.loopq_timing_enable(True)
    lq.loopq_timing_read(5)
    t0 = time.perf_counter()
    for _ in range(steps):
        hessian_step(lq, mods)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    kms, kn = lq.loopq_timing_read(5)[lq.LOOPQ_KERNEL_HESSIAN]
    lq.loopq_timing_enable(False)
    per_k = {}
    for m in mods:  # per input shape, timed alone with the hooks
        lq.loopq_timing_read(5)
        lq.loopq_timing_enable(True)
        for _ in range(steps):
            lq.loopq_hessian_accumulate(m.xt, m.H, m.ws_h)
        torch.cuda.synchronize()
        ms, n = lq.loopq_timing_read(5)[lq.LOOPQ_KERNEL_HESSIAN]
        lq.loopq_timing_enable(False)
        fl = T * M * m.K * (m.K + 1.0)
        per_k[m.act] = {"K": m.K, "rows": T * M, "ms": ms / n, "tflops": fl / (ms / n * 1e-3) / 1e12,
                        "frac": fl / (ms / n * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS}
    flops = sum(T * M * m.K * (m.K + 1.0) for m in mods)
    achieved = flops / (kms / steps * 1e-3) / 1e12
    for m in mods:
        del m.xt, m.H, m.ws_h
    torch.cuda.empty_cache()
    return {
        "what": "H += x~^T x~ over the x~ of all T loops, one call per quantized input (fp32 MFMA SYRK)",
        "ms_per_step": dt * 1e3,
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "kernel_ms_per_step": kms / steps,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / FP32_MFMA_PEAK_TFLOPS,
                     "traffic": hessian_traffic(),
                     "traffic_unit": "fabric bytes per step (FETCH_SIZE + WRITE_SIZE, copy-calibrated, "
                                     "both kernels, all 4 inputs)",
                     "alg_bytes_per_step": sum(4.0 * T * M * m.K + 8.0 * m.K * m.K for m in mods)},
        "per_input": per_k,
    }


def cpu_baseline(wl, mods_meta, rows_hint):
    """The oracle, untuned, on a bounded sample: `rows` token rows of loop 0
    of every quantized input (transform + Eq.(4) RTN + integer group dots +
    rescale), timed on the host; reported as TOPS of the same algorithmic ops."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle
    from bit_ptq_looped_amd import synth

    rows = rows_hint or 256
    prepared = []
    for act, K, lins in mods_meta:
        W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        qw, sw = oracle.quant_weights(W, wl.group_w)       # offline step, not timed
        P1, P2 = synth.factors_for(wl, act, K)
        _, x32 = synth.activations_for(wl, act, K, rows=rows)
        clip = float(synth.clips_for(wl, act)[0])
        prepared.append((x32[0], P1, P2, clip, qw, sw))
    import contextlib
    import os as _os
    import platform

    def timed_run(threads):
        ctx = threadpool_limits(limits=threads) if threadpool_limits else contextlib.nullcontext()
        with ctx:
            t0 = time.perf_counter()
            for x, P1, P2, clip, qw, sw in prepared:
                oracle.linear(x, P1, P2, clip, wl.bits_a, qw, sw, wl.group_w)
            return time.perf_counter() - t0

    ops = sum(2.0 * rows * x.shape[1] * qw.shape[0] for x, _, _, _, qw, _ in prepared)
    dt = timed_run(1)
    ncpu = len(_os.sched_getaffinity(0)) if hasattr(_os, "sched_getaffinity") else (_os.cpu_count() or 1)
    dt_all = timed_run(ncpu)
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = ""
    try:
        from threadpoolctl import threadpool_info
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        pass
    sample = (f"{rows} token rows of loop 0 of each quantized input (qkv, o, up, down) at full K and N; "
              f"weight quantization and input drawing not timed; host {cpu}, numpy {np.__version__}, BLAS {blas}")
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"{sample}; {dt:.1f} s with BLAS limited to 1 thread", "seconds": dt,
            "all_cores": {"value": ops / dt_all / 1e12, "unit": "TOPS", "cores": ncpu, "kind": "oracle",
                          "sample": f"the same sample, BLAS on {ncpu} threads: {dt_all:.1f} s", "seconds": dt_all}}


def calibration_copy(args, torch):
    """One plain device copy of --copy-mib MiB: the reference kernel that
    scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    if not args.copy_mib:
        return
    src = torch.empty(args.copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {args.copy_mib} MiB", flush=True)
    del src, dst


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU; multi-GPU sharding is described, not built "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from bit_ptq_looped_amd import loopq as lq
    from bit_ptq_looped_amd import synth

    lq.load()
    torch.cuda.set_device(0)
    wl = synth.ouro_block_workload(bits_a=4, M=args.M, T=args.T)
    mods = build_modules(lq, synth, wl, torch)
    T, M = wl.T, wl.M
    for m in mods:
        m.y = torch.empty((T, M, m.N), dtype=torch.float32, device="cuda")
        # one workspace serves the W4A4 and W4A8 runs: the larger of the two
        need = max(lq.loopq_workspace_bytes(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, m.K, m.N, b) for b in (4, 8))
        m.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    if args.profile_decode:
        _, dmods = build_decode(lq, synth, torch, 1, 4)
        torch.cuda.synchronize()
        for i in range(args.profile_decode):
            decode_loop_step(lq, dmods, i % 4)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_decode} decode loop-steps", flush=True)
        return
    if args.profile_hessian:
        calibration_copy(args, torch)
        hessian_setup(lq, torch, mods, T, M)
        for _ in range(args.profile_hessian):
            hessian_step(lq, mods)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_hessian} trajectory Hessian steps", flush=True)
        return
    if args.profile_steps:
        calibration_copy(args, torch)
        run_steps(lq, mods, 4, args.profile_schedule, args.profile_steps)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_steps} steps", flush=True)
        return

    ops = alg_ops(mods, T, M)
    s_ws, kern = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_AUTO, args.steps, args.warmup, hooks=True)
    s_ws_nohook, _ = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_AUTO, args.steps, args.warmup)
    s_seq, _ = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_LOOP_SEQUENTIAL, args.steps, args.warmup)
    s_a8, kern_a8 = timed(lq, torch, mods, 8, lq.LOOPQ_SCHED_AUTO, args.steps, args.warmup, hooks=True)

    gemm_ms, gemm_n = kern[lq.LOOPQ_KERNEL_GEMM]
    quant_ms, quant_n = kern[lq.LOOPQ_KERNEL_QUANT_TRANSFORM]
    gemm_ops_total = ops * args.steps
    achieved = gemm_ops_total / (gemm_ms * 1e-3) / 1e12
    bytes_ls = alg_bytes_per_loop_step(mods, M, wl.group_w)

    out = {
        "metric": METRIC,
        "value": ops / s_ws_nohook / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s_ws_nohook * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 codes as e2m3 fp6 MFMA operands, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "M": M, "T": T, "hidden": 2048, "intermediate": 5632,
            "linears": "q|k|v fused (2048->6144), o 2048->2048, up 2048->5632, down 5632->2048",
            "bits": "W4A4", "group_a": 32, "group_w": 32,
            "factors": "(32,64) for K=2048, (64,88) for K=5632",
            "schedule": "weight-stationary (all T loops per launch)",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": achieved / INT8_PEAK_TOPS,
            "traffic": measured_traffic(),
            "traffic_unit": "HBM bytes per GEMM launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "gemm_f6_kernel<0> (W4A4 GEMM on e2m3 MFMA operands + per-group rescale)",
            "frac_fold_inclusive": fold_inclusive(mods, T, M, gemm_ms / args.steps)["frac"],
            "frac_fold_inclusive_note": ("the GEMM kernel time against MFMA time at 5 POPS plus the per-group fold "
                                         "(2 fp32 VALU lane operations per element-group at 39.3 T/s); see "
                                         "fold_inclusive"),
            "launches": gemm_n,
            "avg_launch_ms": gemm_ms / max(gemm_n, 1),
        },
        "ms_per_loop_step": s_ws_nohook * 1e3 / T,
        "tops_per_loop_step": ops / s_ws_nohook / 1e12,
        "gbps_per_loop_step": bytes_ls / (s_ws_nohook / T) / 1e9,
        "frac_int8_peak": ops / s_ws_nohook / 1e12 / INT8_PEAK_TOPS,
        "frac_hbm_peak": bytes_ls / (s_ws_nohook / T) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms_per_step": {"quant_transform": quant_ms / args.steps, "gemm": gemm_ms / args.steps},
        "fold_inclusive": fold_inclusive(mods, T, M, gemm_ms / args.steps),
        "ms_per_step_with_timing_hooks": s_ws * 1e3,
        "loop_sequential_pipelined": {"ms_per_step": s_seq * 1e3, "value": ops / s_seq / 1e12},
        "w4a8": {"ms_per_step": s_a8 * 1e3, "value": ops / s_a8 / 1e12,
                 "gemm_ms_per_step": kern_a8[lq.LOOPQ_KERNEL_GEMM][0] / args.steps},
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_loop_dependent:
        out["loop_dependent"] = loop_dependent_bench(lq, synth, torch, wl, mods, max(5, args.steps // 2), 2)
    if not args.no_per_token:
        out["per_token"] = per_token_bench(lq, torch, mods, T, M, max(5, args.steps // 2), 2)
    if not args.no_hessian:
        out["trajectory_hessian"] = hessian_bench(lq, torch, mods, T, M, max(5, args.steps // 5), 2)
    if not args.no_recurrence:
        out["recurrence"] = [recurrence_bench(lq, synth, torch, 1, 32, 20),
                             recurrence_bench(lq, synth, torch, 2048, 32, 2)]
    if not args.no_decode:
        del mods
        torch.cuda.empty_cache()
        out["decode"] = [decode_bench(lq, synth, torch, Md, 4, args.decode_steps) for Md in (1, 4, 16)]
    if not args.no_cpu_baseline:
        groups = {}
        for lin in wl.linears:
            groups.setdefault(lin.act, []).append(lin)
        meta = [(act, lins[0].K, lins) for act, lins in groups.items()]
        cb = cpu_baseline(wl, meta, args.cpu_rows)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        out["cpu_baseline_all_cores"] = {k: cb["all_cores"][k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
