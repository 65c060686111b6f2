#!/usr/bin/env python3
"""Throughput of the looped W4A4 group-quantized linear on one MI355X.

Headline workload: a 2.6B-like looped stack (hidden 2560, MLP 6912, 48
shared layers, M = 8192 token rows, T loops, W4A4 with groups of 32, Kronecker
factors (40, 64) and (64, 108), one LAS clip per layer, input and loop).  A
step is one looped forward of the whole stack, in the order a looped model
runs it: for each loop t, the 48 layers in turn, and in each layer its four
quantized inputs (q|k|v fused 2560 -> 7680, o 2560 -> 2560, up 2560 -> 6912,
down 6912 -> 2560), each one ``loopq_looped_forward`` call over M rows: the
fused Kronecker transform + group RTN quantizer, then the integer GEMM with
per-group rescale, against that layer's packed INT4 weights, which are the
same at every loop.  Inputs (bf16 activations, packed weights, factors) are
resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--T 4] [--no-cpu-baseline]

Prints one JSON line.  ``value`` is algorithmic GEMM ops (2 M N K summed over
the step's linears, layers and loops) per second of wall time, in TOPS; the
same figure per loop-step is ``tops_per_loop_step``, and ``t_sweep`` repeats
it for T = 1, 2, 4, 8.  Secondary lines: the Ouro-1.4B-like block (M = 1024,
T = 4, W4A4 and W4A8, loop-dependent sets, per-token steps, trajectory
Hessian), the Huginn-like core linears and adapter recurrence, and the
decode stack.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "looped W4A4 linear TOPS & GB/s per loop-step, % of INT8-MFMA/HBM roofline"
INT8_PEAK_TOPS = 5000.0          # MI355X dense INT8 MFMA, 5.0 POP/s
FP6_PEAK_TFLOPS = 10100.0        # MI355X dense fp6 / fp4 MFMA, 10.1 PFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix
# the trajectory Hessian takes each multiply-add as six bf16-plane products
HESSIAN_PEAK_TFLOPS = BF16_MFMA_PEAK_TFLOPS / 6.0
FP32_VALU_PEAK_TFLOPS = 157.3    # MI355X fp32 vector (an FMA counts two flops)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
STACK_LAYERS = 48
STACK_DRAWN_LOOPS = 4            # loop inputs drawn on the host; loop t reads input t mod 4
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--T", type=int, default=4, help="loops of the headline step")
    p.add_argument("--M", type=int, default=8192, help="token rows of the headline stack")
    p.add_argument("--layers", type=int, default=STACK_LAYERS)
    p.add_argument("--sweep", default="1,2,4,8", help="loop counts of the T sweep ('' to skip)")
    p.add_argument("--sweep-steps", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=256, help="token rows in the oracle sample")
    p.add_argument("--no-stack", action="store_true",
                   help="skip the headline stack (development runs of the secondary lines; value is then null)")
    p.add_argument("--no-block", action="store_true", help="skip the Ouro-1.4B-like block lines")
    p.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    p.add_argument("--no-loop-dependent", action="store_true",
                   help="skip the loop-dependent (per-loop weight sets / bit widths) measurement")
    p.add_argument("--no-hessian", action="store_true", help="skip the trajectory Hessian measurement")
    p.add_argument("--no-recurrence", action="store_true", help="skip the adapter recurrence measurement")
    p.add_argument("--no-per-token", action="store_true", help="skip the per-token measurement")
    p.add_argument("--no-cta", action="store_true", help="skip the CTA adapter measurement")
    p.add_argument("--no-huginn-core", action="store_true", help="skip the Huginn-like core linears")
    p.add_argument("--profile-stack", type=int, default=0,
                   help="only run this many headline steps (for rocprofv3), no JSON")
    p.add_argument("--profile-steps", type=int, default=0,
                   help="only run this many steps of the Ouro-like block (for rocprofv3), no JSON")
    p.add_argument("--profile-schedule", type=int, default=0,
                   help="schedule used by --profile-steps (0 auto, 1 loop-sequential, 2 weight-stationary)")
    p.add_argument("--profile-hessian", type=int, default=0,
                   help="only run this many trajectory Hessian steps (for a profiler) and exit")
    p.add_argument("--decode-steps", type=int, default=20)
    p.add_argument("--profile-decode", type=int, default=0,
                   help="only run this many decode loop-steps at M=1 (for rocprofv3), no JSON")
    p.add_argument("--profile-reuse", type=int, default=0,
                   help="only run this many rounds of the decode weight-reuse call (layer 0, all T = 4 loops "
                        "of M = 1 in one weight-stationary call per input, the L2 flushed by a 128 MiB copy "
                        "before each), for rocprofv3 FETCH_SIZE; no JSON")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="with a --profile-* run: first run one device-to-device copy of this many MiB "
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


def groups_by_input(wl):
    groups = {}
    for lin in wl.linears:
        groups.setdefault(lin.act, []).append(lin)
    return groups


# ---------------------------------------------------------------------------
# the bound of the W4A4 GEMM that counts the per-group fold
# ---------------------------------------------------------------------------

def fold_inclusive(ops, element_groups, gemm_ms):
    """The GEMM against a bound that counts the per-group fold the method
    requires (y = sum_j s_a s_w d_j): per element-group, the kernel forms the
    step product s_a * s_w on the fp32 outer-product MFMA (one multiply-add)
    and folds it with one fp32 FMA on the VALU, besides the integer MFMA work.
    On gfx950 the MFMA and VALU issue cycles of one SIMD add up (measured),
    so the bound is the sum of the three times at their dense peaks: the
    integer ops at 5.0 POP/s, the coefficient multiply-adds at the fp32 MFMA's
    157.3 / 2 T/s and the FMAs at the fp32 VALU's 157.3 / 2 T/s."""
    t_mfma = ops / (INT8_PEAK_TOPS * 1e12)
    t_coef = element_groups / (FP32_MFMA_PEAK_TFLOPS * 1e12 / 2)
    t_fma = element_groups / (FP32_VALU_PEAK_TFLOPS * 1e12 / 2)
    bound = t_mfma + t_coef + t_fma
    return {"element_groups": element_groups, "t_mfma_ms": t_mfma * 1e3, "t_coef_ms": t_coef * 1e3,
            "t_fma_ms": t_fma * 1e3, "bound_ms": bound * 1e3, "gemm_ms": gemm_ms,
            "bound_tops": ops / bound / 1e12, "frac": bound * 1e3 / gemm_ms if gemm_ms > 0 else None}


def timing_read(lq, n=7):
    return lq.loopq_timing_read(n)


def median_blocks(torch, lq, run, steps, blocks=3):
    """Wall time per step of run(steps), as `blocks` separately timed blocks,
    each also with the summed kernel time of its launches (timing hooks on):
    (median seconds per step, per-block wall ms per step, per-block kernel ms
    per step).  A block whose wall time is far above its kernel time lost the
    difference between launches (host side), one whose kernel time rose lost
    it on the GPU."""
    walls, kerns = [], []
    for _ in range(blocks):
        torch.cuda.synchronize()
        lq.loopq_timing_reset()
        lq.loopq_timing_enable(True)
        t0 = time.perf_counter()
        run(steps)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) / steps)
        lq.loopq_timing_enable(False)
        kerns.append(sum(ms for ms, _ in timing_read(lq)) / steps)
    return (sorted(walls)[len(walls) // 2], [round(w * 1e3, 4) for w in walls],
            [round(k, 4) for k in kerns])


# ---------------------------------------------------------------------------
# the headline: the 2.6B-like looped stack
# ---------------------------------------------------------------------------

def build_stack(lq, synth, torch, M, layers):
    """Per quantized input: factors, the drawn loop inputs [4][M][K] (bf16),
    clips [layers][8] and packed weights for every layer.  Layer 0 packs the
    seeded fp32 weights; deeper layers get seeded random packed bytes and fp16
    steps drawn on the device (kernel time does not depend on the values;
    parity runs on layer 0)."""
    import numpy as np
    wl = synth.large_prefill_workload(T=STACK_DRAWN_LOOPS, M=M, layers=layers)
    wl8 = synth.large_prefill_workload(T=8, M=M, layers=layers)  # clips of up to 8 loops
    gen = torch.Generator(device="cuda")
    gen.manual_seed(26_048)
    mods = []
    for act, lins in groups_by_input(wl).items():
        K = lins[0].K
        W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        N = W.shape[0]
        P1, P2 = synth.factors_for(wl, act, K)
        bits, _ = synth.activations_for(wl, act, K)
        x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)  # [4][M][K]
        del bits
        weights = []
        for layer in range(layers):
            codes, scales = lq.empty_packed_weights(K, N, wl.group_w)
            if layer == 0:
                lq.loopq_pack_weights(torch.from_numpy(W).cuda(), wl.group_w, codes, scales)
            else:
                codes.copy_(torch.randint(0, 256, codes.shape, dtype=torch.uint8, device="cuda", generator=gen))
                steps = torch.rand(scales.numel() // 2, device="cuda", generator=gen) * 0.004 + 0.001
                scales.copy_(steps.to(torch.float16).view(torch.uint8))
            weights.append((codes, scales))
        m = Module(act, K, N, torch.from_numpy(P1).cuda(), torch.from_numpy(P2).cuda(),
                   [[float(c) for c in synth.clips_for(wl8, act, layer)] for layer in range(layers)], x, None, None)
        m.weights = weights
        m.views = [x[t:t + 1] for t in range(STACK_DRAWN_LOOPS)]
        m.y = torch.empty((1, M, N), dtype=torch.float32, device="cuda")
        m.ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, 1, M, K, N, 4)
        mods.append(m)
    torch.cuda.synchronize()
    return wl, mods


def stack_step(lq, mods, T, layers):
    """One looped forward of the stack, loop by loop (a looped model's order)."""
    for t in range(T):
        for layer in range(layers):
            for m in mods:
                codes, scales = m.weights[layer]
                lq.loopq_looped_forward(m.views[t % STACK_DRAWN_LOOPS], m.P1, m.P2, [m.clips[layer][t]], 4, codes,
                                        scales, 32, m.N, m.y, lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.ws)


def stack_step_ws(lq, mods, T, layers):
    """The same work with each layer's T loops batched into one call per
    input (T * M rows against the layer's weights; independent loop inputs)."""
    for layer in range(layers):
        for m in mods:
            codes, scales = m.weights[layer]
            lq.loopq_looped_forward(m.xT, m.P1, m.P2, m.clips[layer][:T], 4, codes, scales, 32, m.N, m.yT,
                                    lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.wsT)


def stack_ops_per_loop(mods, M, layers):
    return layers * sum(2.0 * M * m.N * m.K for m in mods)


def stack_groups_per_loop(mods, M, layers):
    return layers * sum(M * m.N * m.K / 32.0 for m in mods)


def stack_bytes_per_loop(mods, M, layers):
    """Packed weights + fp16 steps + bf16 activations in + fp32 y out, per loop-step."""
    return layers * sum(m.N * m.K / 2 + 2 * m.N * (m.K // 32) + 2 * M * m.K + 4 * M * m.N for m in mods)


def time_loop(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


STACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_stack_2p6b_M8192.md")
BLOCK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_ouro_block_M1024_T4.md")


def gemm_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ("bit_ptq_looped_amd/csrc/gemm_f6.hip", "bit_ptq_looped_amd/csrc/gemm_tile.h"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(path):
    """HBM bytes per GEMM launch from a committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the GEMM source changed since it was taken."""
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines() if line.startswith("gemm_"))
    except OSError:
        return None
    if fields.get("gemm_source_sha256") != gemm_source_sha256():
        return None
    return float(fields["gemm_traffic_bytes_per_launch"])


def stack_bench(lq, synth, torch, args):
    M, L, T = args.M, args.layers, args.T
    wl, mods = build_stack(lq, synth, torch, M, L)
    ops_loop = stack_ops_per_loop(mods, M, L)
    bytes_loop = stack_bytes_per_loop(mods, M, L)
    groups_loop = stack_groups_per_loop(mods, M, L)
    dt = time_loop(torch, lambda: stack_step(lq, mods, T, L), args.steps, args.warmup)
    # the same steps with the timing hooks: per-kernel time and GEMM launches
    lq.loopq_timing_reset()
    lq.loopq_timing_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        stack_step(lq, mods, T, L)
    torch.cuda.synchronize()
    dt_hooks = (time.perf_counter() - t0) / args.steps
    lq.loopq_timing_enable(False)
    kern = timing_read(lq)
    gemm_ms, gemm_n = kern[lq.LOOPQ_KERNEL_GEMM]
    quant_ms, quant_n = kern[lq.LOOPQ_KERNEL_QUANT_TRANSFORM]
    ops_step = ops_loop * T
    achieved = ops_step * args.steps / (gemm_ms * 1e-3) / 1e12
    fi = fold_inclusive(ops_step, groups_loop * T, gemm_ms / args.steps)
    res = {
        "wl": wl, "mods": mods, "dt": dt, "ops_step": ops_step, "bytes_loop": bytes_loop,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": achieved / INT8_PEAK_TOPS,
            "traffic": measured_traffic(STACK_TRAFFIC_FILE),
            "traffic_unit": "HBM bytes per GEMM launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated; mean over the "
                            "four layer linears)",
            "kernel": "gemm_f6_kernel<0> (W4A4 GEMM on e2m3 fp6 MFMA operands + per-group rescale), M = 8192 rows "
                      "per launch",
            "launches": gemm_n,
            "avg_launch_ms": gemm_ms / max(gemm_n, 1),
            "alg_ops_per_launch": ops_step * args.steps / max(gemm_n, 1),
            "frac_fp6_peak": achieved / FP6_PEAK_TFLOPS,
            "fp6_peak": FP6_PEAK_TFLOPS,
            "frac_fold_inclusive": fi["frac"],
            "fold_inclusive_bound_tops": fi["bound_tops"],
        },
        "kernels_ms_per_step": {"quant_transform": quant_ms / args.steps, "gemm": gemm_ms / args.steps,
                                "launches_per_step": {"quant_transform": quant_n / args.steps,
                                                      "gemm": gemm_n / args.steps}},
        "fold_inclusive": fi,
        "ms_per_step_with_timing_hooks": dt_hooks * 1e3,
    }
    # T sweep: per loop-step throughput at T = 1, 2, 4, 8, loop by loop (the
    # headline order) and with each layer's loops batched into one call
    sweep = []
    Ts = [int(v) for v in args.sweep.split(",") if v.strip()] if args.sweep else []
    for Ts_ in Ts:
        d_ls = time_loop(torch, lambda: stack_step(lq, mods, Ts_, L), args.sweep_steps, 1)
        for m in mods:
            m.xT = torch.cat([m.x[t % STACK_DRAWN_LOOPS:t % STACK_DRAWN_LOOPS + 1] for t in range(Ts_)], 0)
            m.yT = torch.empty((Ts_, M, m.N), dtype=torch.float32, device="cuda")
            m.wsT = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, Ts_, M, m.K, m.N, 4)
        d_ws = time_loop(torch, lambda: stack_step_ws(lq, mods, Ts_, L), args.sweep_steps, 1)
        for m in mods:
            del m.xT, m.yT, m.wsT
        torch.cuda.empty_cache()
        sweep.append({"T": Ts_,
                      "loop_sequential": {"ms_per_step": d_ls * 1e3, "ms_per_loop_step": d_ls * 1e3 / Ts_,
                                          "tops_per_loop_step": ops_loop * Ts_ / d_ls / 1e12},
                      "weight_stationary": {"ms_per_step": d_ws * 1e3, "ms_per_loop_step": d_ws * 1e3 / Ts_,
                                            "tops_per_loop_step": ops_loop * Ts_ / d_ws / 1e12,
                                            "rows_per_launch": Ts_ * M}})
    res["t_sweep"] = sweep
    return res


# ---------------------------------------------------------------------------
# the Ouro-1.4B-like block (M = 1024, T = 4): secondary lines
# ---------------------------------------------------------------------------

def build_modules(lq, synth, wl, torch):
    """Group the block's linears by quantized input (q, k, v share qkv_in and
    are packed as one weight of N = 3 * hidden), draw inputs, pack weights."""
    import numpy as np
    mods = []
    for act, lins in groups_by_input(wl).items():
        K = lins[0].K
        W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        N = W.shape[0]
        codes, scales = lq.empty_packed_weights(K, N, wl.group_w)
        lq.loopq_pack_weights(torch.from_numpy(W).cuda(), wl.group_w, codes, scales)
        P1, P2 = synth.factors_for(wl, act, K)
        bits, _ = synth.activations_for(wl, act, K)
        x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        mods.append(Module(act, K, N, torch.from_numpy(P1).cuda(), torch.from_numpy(P2).cuda(),
                           [float(c) for c in synth.clips_for(wl, act)], x, codes, scales))
    return mods


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
    per_kernel = timing_read(lq)
    return (t1 - t0) / steps, per_kernel


def graph_step_ms(lq, torch, mods, bits, schedule, steps):
    """One step of the block captured into a HIP graph (the pipelined schedule's
    auxiliary stream and events become graph nodes), replayed three times with
    eager work between the replays and every replay's outputs checked bitwise
    against an eager step, then timed over `steps` replays.  Returns (ms per
    step or None, replays match, error text or None)."""
    run_steps(lq, mods, bits, schedule, 1)
    torch.cuda.synchronize()
    ref = [m.y.clone() for m in mods]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    try:
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                run_steps(lq, mods, bits, schedule, 1)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
    except Exception as e:  # capture is a measurement option, not part of the path
        torch.cuda.synchronize()
        return None, False, str(e)[:200]
    ok = True
    for _ in range(3):
        for m in mods:
            m.y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        ok &= all(torch.equal(m.y, r) for m, r in zip(mods, ref))
        run_steps(lq, mods, bits, schedule, 1)  # eager work between replays
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    del graph
    return dt * 1e3, bool(ok), None


def setup_block(lq, synth, torch, M=1024, T=4):
    wl = synth.ouro_block_workload(bits_a=4, M=M, T=T)
    mods = build_modules(lq, synth, wl, torch)
    for m in mods:
        m.y = torch.empty((T, M, m.N), dtype=torch.float32, device="cuda")
        # one workspace serves the W4A4 and W4A8 runs: the larger of the two
        need = max(lq.loopq_workspace_bytes(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, m.K, m.N, b) for b in (4, 8))
        m.ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    return wl, mods


def block_bench(lq, torch, wl, mods, steps, warmup):
    T, M = wl.T, wl.M
    ops = alg_ops(mods, T, M)
    s_ws, kern = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_AUTO, steps, warmup, hooks=True)
    s_ws_nohook, _ = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_AUTO, steps, warmup)
    s_seq, kern_seq = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_LOOP_SEQUENTIAL, steps, warmup, hooks=True)
    s_seq_nohook, _ = timed(lq, torch, mods, 4, lq.LOOPQ_SCHED_LOOP_SEQUENTIAL, steps, warmup)
    s_a8, kern_a8 = timed(lq, torch, mods, 8, lq.LOOPQ_SCHED_AUTO, steps, warmup, hooks=True)
    g_ws = graph_step_ms(lq, torch, mods, 4, lq.LOOPQ_SCHED_AUTO, steps)
    g_seq = graph_step_ms(lq, torch, mods, 4, lq.LOOPQ_SCHED_LOOP_SEQUENTIAL, steps)
    gemm_ms, gemm_n = kern[lq.LOOPQ_KERNEL_GEMM]
    quant_ms, _ = kern[lq.LOOPQ_KERNEL_QUANT_TRANSFORM]
    achieved = ops * steps / (gemm_ms * 1e-3) / 1e12
    groups = sum(T * M * m.N * m.K / 32.0 for m in mods)
    seq_gemm_ms, seq_gemm_n = kern_seq[lq.LOOPQ_KERNEL_GEMM]
    bytes_ls = alg_bytes_per_loop_step(mods, M, wl.group_w)
    return {
        "workload": wl.name,
        "what": "per quantized input (q|k|v fused 2048->6144, o, up 2048->5632, down 5632->2048): all T loops "
                "in one weight-stationary call (T*M = 4096 rows per GEMM launch)",
        "ms_per_step": s_ws_nohook * 1e3,
        "value": ops / s_ws_nohook / 1e12,
        "unit": "TOPS",
        "gbps_per_loop_step": bytes_ls / (s_ws_nohook / T) / 1e9,
        "kernels_ms_per_step": {"quant_transform": quant_ms / steps, "gemm": gemm_ms / steps},
        "gemm": {"achieved_tops": achieved, "frac_int8_peak": achieved / INT8_PEAK_TOPS,
                 "frac_fp6_peak": achieved / FP6_PEAK_TFLOPS, "avg_launch_ms": gemm_ms / max(gemm_n, 1),
                 "launches": gemm_n, "traffic": measured_traffic(BLOCK_TRAFFIC_FILE)},
        "fold_inclusive": fold_inclusive(ops, groups, gemm_ms / steps),
        "ms_per_step_with_timing_hooks": s_ws * 1e3,
        "graph_ms_per_step": g_ws[0], "graph_replays_match_eager": g_ws[1], "graph_error": g_ws[2],
        "loop_sequential_pipelined": {
            "graph_ms_per_step": g_seq[0], "graph_replays_match_eager": g_seq[1], "graph_error": g_seq[2],
            "ms_per_step": s_seq_nohook * 1e3, "value": ops / s_seq_nohook / 1e12,
            "gemm_launches": seq_gemm_n,
            "gemm_avg_launch_ms": seq_gemm_ms / max(seq_gemm_n, 1),
            "gemm_achieved_tops": ops * steps / (seq_gemm_ms * 1e-3) / 1e12,
            "ms_per_step_with_timing_hooks": s_seq * 1e3},
        "w4a8": {"ms_per_step": s_a8 * 1e3, "value": ops / s_a8 / 1e12,
                 "gemm_ms_per_step": kern_a8[lq.LOOPQ_KERNEL_GEMM][0] / steps,
                 "gemm_achieved_tops": ops * steps / (kern_a8[lq.LOOPQ_KERNEL_GEMM][0] * 1e-3) / 1e12},
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
        dt, walls, kerns = median_blocks(torch, lq, lambda n: run(kind, n), steps)
        out[kind] = {"ms_per_step": dt * 1e3, "value": ops / dt / 1e12, "blocks_ms_per_step": walls,
                     "blocks_kernel_ms_per_step": kerns}
    out["slt"]["what"] = ("every loop with its own packed weights and factors (no sharing): per input, one "
                          "quantizer launch per loop and one grouped GEMM over all T*M rows")
    out["bits_8444"]["what"] = "loop 0 at A8, loops 1-3 at A4, shared weights: two weight-stationary runs per input"
    for m in mods:
        del m.own_weights, m.own_factors, m.ws_ex
    return out


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
    dt, walls, kerns = median_blocks(torch, lq, run, steps)
    for m in mods:
        del m.ws_tok
    return {"what": "per-token activation steps, W4A4, all T loops of an input in one weight-stationary call",
            "ms_per_step": dt * 1e3, "value": alg_ops(mods, T, M) / dt / 1e12, "unit": "TOPS",
            "blocks_ms_per_step": walls, "blocks_kernel_ms_per_step": kerns}


HESSIAN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_trajectory_hessian_ouro_block_M1024_T4.md")


def hessian_traffic():
    """Counter bytes per trajectory Hessian step from the committed summary,
    or None when hessian.hip changed since the counters were taken."""
    import hashlib
    try:
        fields = dict(line.split(": ", 1) for line in open(HESSIAN_TRAFFIC_FILE).read().splitlines()
                      if line.startswith("hessian_"))
        with open(os.path.join(ROOT, "bit_ptq_looped_amd/csrc/hessian.hip"), "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
    except OSError:
        return None
    if fields.get("hessian_source_sha256") != sha:
        return None
    return float(fields["hessian_traffic_bytes_per_step"])


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


def hessian_side_bench(lq, torch, mods, T, M, steps):
    """The looped forward with the trajectory Hessian as its side output
    (loopq_looped_forward_hessian: the forward's quantizer writes x~, then the
    SYRK) against the separate path: loopq_quant_act for the x~ dump, the
    forward, then loopq_hessian_accumulate.  Weight-stationary, every
    quantized input of the block, T*M rows each."""
    WS = lq.LOOPQ_SCHED_WEIGHT_STATIONARY
    bufs = []
    for m in mods:
        rows = T * m.x.shape[1]
        b = {"ws": lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_HESSIAN, T, M, m.K, m.N, 4),
             "ws_f": lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, m.K, m.N, 4),
             "ws_h": lq.empty_workspace(lq.LOOPQ_OP_HESSIAN, 0, rows, m.K, 0, 0),
             "H": torch.zeros((m.K, m.K), dtype=torch.float32, device="cuda"),
             "y": torch.empty((T, M, m.N), dtype=torch.float32, device="cuda"),
             "codes": torch.empty((rows, m.K), dtype=torch.int8, device="cuda"),
             "steps": torch.empty((rows, m.K // 32), dtype=torch.float32, device="cuda"),
             "xt": torch.empty((rows, m.K), dtype=torch.float32, device="cuda")}
        bufs.append(b)

    def side(n):
        for _ in range(n):
            for m, b in zip(mods, bufs):
                lq.loopq_looped_forward_hessian(m.x, m.P1, m.P2, m.clips[:T], 4, m.codes, m.scales, 32, m.N, b["y"],
                                                WS, b["H"], b["ws"])

    def separate(n):
        for _ in range(n):
            for m, b in zip(mods, bufs):
                lq.loopq_quant_act(m.x.reshape(T * M, m.K), m.P1, m.P2, 1.0, 4, b["codes"], b["steps"], b["xt"])
                lq.loopq_looped_forward(m.x, m.P1, m.P2, m.clips[:T], 4, m.codes, m.scales, 32, m.N, b["y"], WS,
                                        b["ws_f"])
                lq.loopq_hessian_accumulate(b["xt"], b["H"], b["ws_h"])

    side(1)
    separate(1)
    t_side, walls_s, kern_s = median_blocks(torch, lq, side, steps)
    t_sep, walls_p, kern_p = median_blocks(torch, lq, separate, steps)
    del bufs
    torch.cuda.empty_cache()
    return {"what": "looped forward + trajectory Hessian per step (all 4 quantized inputs, weight-stationary): "
                    "one loopq_looped_forward_hessian call per input vs quantizer dump + forward + accumulation",
            "side_output_ms_per_step": t_side * 1e3, "separate_ms_per_step": t_sep * 1e3,
            "saving_frac": (t_sep - t_side) / t_sep,
            "blocks_ms": {"side_output": walls_s, "separate": walls_p},
            "blocks_kernel_ms": {"side_output": kern_s, "separate": kern_p}}


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
    timing_read(lq)
    t0 = time.perf_counter()
    for _ in range(steps):
        hessian_step(lq, mods)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    kms, kn = timing_read(lq)[lq.LOOPQ_KERNEL_HESSIAN]
    lq.loopq_timing_enable(False)
    per_k = {}
    for m in mods:  # per input shape, timed alone with the hooks
        timing_read(lq)
        lq.loopq_timing_enable(True)
        for _ in range(steps):
            lq.loopq_hessian_accumulate(m.xt, m.H, m.ws_h)
        torch.cuda.synchronize()
        ms, n = timing_read(lq)[lq.LOOPQ_KERNEL_HESSIAN]
        lq.loopq_timing_enable(False)
        fl = T * M * m.K * (m.K + 1.0)
        per_k[m.act] = {"K": m.K, "rows": T * M, "ms": ms / n, "tflops": fl / (ms / n * 1e-3) / 1e12,
                        "frac": fl / (ms / n * 1e-3) / 1e12 / HESSIAN_PEAK_TFLOPS,
                        "frac_fp32_mfma_peak": fl / (ms / n * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS}
    flops = sum(T * M * m.K * (m.K + 1.0) for m in mods)
    achieved = flops / (kms / steps * 1e-3) / 1e12
    for m in mods:
        del m.xt, m.H, m.ws_h
    torch.cuda.empty_cache()
    return {
        "what": "H += x~^T x~ over the x~ of all T loops, one call per quantized input (SYRK on the bf16 MFMA, "
                "six exact bf16-plane products per multiply-add, fp32 accumulation)",
        "ms_per_step": dt * 1e3,
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "kernel_ms_per_step": kms / steps,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": HESSIAN_PEAK_TFLOPS,
                     "peak_note": "bf16 dense MFMA rate / 6 (six plane products per algorithmic multiply-add)",
                     "unit": "TFLOP/s", "frac": achieved / HESSIAN_PEAK_TFLOPS,
                     "frac_fp32_mfma_peak": achieved / FP32_MFMA_PEAK_TFLOPS,
                     "traffic": hessian_traffic(),
                     "traffic_unit": "fabric bytes per step (FETCH_SIZE + WRITE_SIZE, copy-calibrated, "
                                     "both kernels, all 4 inputs)",
                     "alg_bytes_per_step": sum(4.0 * T * M * m.K + 8.0 * m.K * m.K for m in mods)},
        "per_input": per_k,
    }


# ---------------------------------------------------------------------------
# the Huginn-like linears (weight groups of 128, A8, no transform)
# ---------------------------------------------------------------------------

HUGINN_BLOCK_ROWS = 256


def cta_bench(lq, synth, torch, steps):
    """CTA at the loop transitions of the 2.6B-like stack's q|k|v input:
    M = 8192 rows, K = 2560, N = 7680, T = 4 loops, bf16 state, rank 8.  The
    adapter kernel runs over all T*M rows of one loopq_looped_forward_cta call
    (loop 0 copied, loops 1..3 adapted); the call is timed against the plain
    loopq_looped_forward (weight-stationary) on the same inputs."""
    M, K, N, T, r = 8192, 2560, 7680, 4, 8
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7007)
    rng = synth.seeded_rng(synth.TEST, 7007)
    x = torch.randn((T, M, K), generator=gen, device="cuda").to(torch.bfloat16)
    U = torch.randn((K, r), generator=gen, device="cuda") / K ** 0.5
    V = torch.randn((K, r), generator=gen, device="cuda") / K ** 0.5
    a = 1.0 + 0.1 * torch.randn((T - 1, K), generator=gen, device="cuda")
    b = 0.05 * torch.randn((T - 1, K), generator=gen, device="cuda")
    eta = [0.3, -0.2, 0.5]
    P1 = torch.from_numpy(synth.haar_orthogonal(40, rng)).cuda()
    P2 = torch.from_numpy(synth.haar_orthogonal(64, rng)).cuda()
    codes, scales = lq.empty_packed_weights(K, N, 32)
    codes.copy_(torch.randint(0, 256, codes.shape, dtype=torch.uint8, device="cuda", generator=gen))
    st = torch.rand(scales.numel() // 2, device="cuda", generator=gen) * 0.004 + 0.001
    scales.copy_(st.to(torch.float16).view(torch.uint8))
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_CTA, T, M, K, N, 4)
    clips = [1.0] * T
    WS = lq.LOOPQ_SCHED_WEIGHT_STATIONARY

    def plain(n):
        for _ in range(n):
            lq.loopq_looped_forward(x, P1, P2, clips, 4, codes, scales, 32, N, y, WS, ws)

    def with_cta(n):
        for _ in range(n):
            lq.loopq_looped_forward_cta(x, P1, P2, clips, 4, codes, scales, 32, N, y, WS, U, V, a, b, eta, ws)

    plain(1)
    with_cta(1)
    t_plain, walls_p, kern_p = median_blocks(torch, lq, plain, steps)
    t_cta, walls_c, kern_c = median_blocks(torch, lq, with_cta, steps)
    lq.loopq_timing_reset()
    lq.loopq_timing_enable(True)
    with_cta(steps)
    torch.cuda.synchronize()
    lq.loopq_timing_enable(False)
    cms, cn = timing_read(lq)[lq.LOOPQ_KERNEL_CTA]
    cta_ms = cms / max(cn, 1)
    # algorithmic bytes of one adapter launch: read and write every row once,
    # plus a, b of each transition and U, V
    alg = 2.0 * T * M * K * 2 + (T - 1) * K * 4 * 2 + 2 * K * r * 4
    out = {"workload": "CTA at the transitions of the 2.6B-like stack's q|k|v input, M=8192, K=2560, N=7680, T=4, "
                       "bf16 state, rank 8, weight-stationary",
           "forward_ms": t_plain * 1e3, "forward_cta_ms": t_cta * 1e3,
           "overhead_frac": (t_cta - t_plain) / t_plain,
           "cta_kernel_ms": cta_ms, "cta_kernel_launches": cn // max(steps, 1),
           "cta_alg_bytes": alg, "cta_gbps": alg / (cta_ms * 1e-3) / 1e9,
           "cta_frac_hbm_peak": alg / (cta_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "blocks_ms": {"forward": walls_p, "forward_cta": walls_c},
           "blocks_kernel_ms": {"forward": kern_p, "forward_cta": kern_c}}
    del x, y, ws, codes, scales
    torch.cuda.empty_cache()
    return out


def huginn_core_bench(lq, synth, torch, steps):
    """The Huginn-like core linears at M = 2048 token rows: Wqkv 5280 -> 15840
    and mlp.proj 17920 -> 5280, weight groups of 128, A8 activations in groups
    of 32, no transform, over T = 32 recurrence steps.  One recurrence step is
    one call per linear (M rows, the step's own clip-1 input); the inputs of
    the 32 steps follow the recurrence x_{t+1} = 0.9 x_t + 0.1 xi_t, drawn as
    a 256-row seeded block repeated along M (rows are independent here)."""
    import numpy as np
    wl = synth.huginn_workload()
    T, M = wl.T, wl.M
    out = []
    for act, name in (("core_in", "wqkv"), ("proj_in", "mlp_proj")):
        lin = [l for l in wl.linears if l.act == act][0]
        K, N, gw = lin.K, lin.N, wl.group_w
        W = synth.weights_for(wl, lin)
        codes, scales = lq.empty_packed_weights(K, N, gw)
        lq.loopq_pack_weights(torch.from_numpy(W).cuda(), gw, codes, scales)
        del W
        bits, _ = synth.activations_for(wl, act, K, rows=HUGINN_BLOCK_ROWS)
        x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16).repeat(1, M // HUGINN_BLOCK_ROWS, 1)
        x = x.contiguous()
        del bits
        views = [x[t:t + 1] for t in range(T)]
        y = torch.empty((1, M, N), dtype=torch.float32, device="cuda")
        ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, 1, M, K, N, 8)

        def step():
            for t in range(T):
                lq.loopq_looped_forward(views[t], None, None, [1.0], 8, codes, scales, gw, N, y,
                                        lq.LOOPQ_SCHED_WEIGHT_STATIONARY, ws)

        dt = time_loop(torch, step, steps, 1)
        lq.loopq_timing_reset()
        lq.loopq_timing_enable(True)
        step()
        torch.cuda.synchronize()
        lq.loopq_timing_enable(False)
        kern = timing_read(lq)
        gms, gn = kern[lq.LOOPQ_KERNEL_GEMM]
        ops = 2.0 * M * N * K * T
        wbytes = codes.numel() + scales.numel()
        out.append({"linear": name, "K": K, "N": N, "M": M, "T": T, "group_w": gw, "bits": "W4A8",
                    "ms_per_recurrence_step": dt * 1e3 / T, "tops": ops / dt / 1e12,
                    "frac_int8_peak": ops / dt / 1e12 / INT8_PEAK_TOPS,
                    "gemm_avg_launch_ms": gms / max(gn, 1),
                    "gemm_achieved_tops": ops / (gms * 1e-3) / 1e12,
                    "quant_ms_per_step": kern[lq.LOOPQ_KERNEL_QUANT_PLAIN][0] / T,
                    "gbps": (wbytes + 2.0 * M * K + 4.0 * M * N) * T / dt / 1e9})
        del x, views, y, ws, codes, scales
        torch.cuda.empty_cache()
    return out


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


# ---------------------------------------------------------------------------
# decode: the Ouro-like block at M <= 16 over 24 layers
# ---------------------------------------------------------------------------

DECODE_LAYERS = 24


def build_decode(lq, synth, torch, M, T, layers=DECODE_LAYERS):
    """The Ouro-like block at decode size: per quantized input, one loop's
    M rows (bf16), the input's factors and clips, and packed weights for
    `layers` distinct layers.  Layer 0 packs the seeded weights; deeper layers
    get seeded random packed bytes and fp16 steps drawn on the device (kernel
    time does not depend on the values; parity runs on layer 0 shapes)."""
    import numpy as np
    wl = synth.ouro_block_workload(bits_a=4, M=M, T=T)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20260)
    mods = []
    for act, lins in groups_by_input(wl).items():
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
    kern = timing_read(lq)
    launches = sum(n for _, n in kern) / steps
    t0 = time.perf_counter()
    for i in range(steps):
        decode_loop_step(lq, mods, i % T)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # the same loop-steps replayed from a captured graph (launch gaps only):
    # loops 0..T-1 once each per replay; outputs checked against eager runs
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
        "kernel_ms_per_loop_step": {
            "decode": kern[lq.LOOPQ_KERNEL_DECODE][0] / steps,
            "transform_and_quantizer": sum(kern[k][0] for k in (lq.LOOPQ_KERNEL_QUANT_TRANSFORM,
                                                                lq.LOOPQ_KERNEL_QUANT_PLAIN)) / steps},
        "kernel_time_note": "summed HIP-event intervals around each launch on its stream (a launch's interval "
                            "includes its queueing behind the previous one, so the sum can exceed the wall time)",
        "launches_per_loop_step": launches,
        "bytes_per_loop_step": step_bytes,
        "graph_ms_per_loop_step": graph_wall * 1e3,
        "graph_gbps_per_loop_step": step_bytes / graph_wall / 1e9,
        "graph_frac_hbm_peak": step_bytes / graph_wall / 1e9 / HBM_PEAK_GBS,
        "graph_replays_match_eager": bool(graph_ok),
        "reuse_one_layer_T_loops_ms": reuse * 1e3,
        "reuse_weight_bytes_per_loop": per_layer_bytes / T,
    }


# ---------------------------------------------------------------------------
# the oracle on the host
# ---------------------------------------------------------------------------

def cpu_baseline(wl, rows):
    """The oracle, untuned, on a bounded sample of the headline workload:
    `rows` token rows of loop 0 of every quantized input of layer 0
    (transform + Eq.(4) RTN + integer group dots + rescale), timed on the
    host; reported as TOPS of the same algorithmic ops."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import contextlib
    import platform

    import oracle
    from bit_ptq_looped_amd import synth

    prepared = []
    for act, lins in groups_by_input(wl).items():
        K = lins[0].K
        W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
        qw, sw = oracle.quant_weights(W, wl.group_w)       # offline step, not timed
        P1, P2 = synth.factors_for(wl, act, K)
        _, x32 = synth.activations_for(wl, act, K, rows=rows)
        clip = float(synth.clips_for(wl, act)[0])
        prepared.append((x32[0], P1, P2, clip, qw, sw))

    def timed_run(threads):
        ctx = threadpool_limits(limits=threads) if threadpool_limits else contextlib.nullcontext()
        with ctx:
            t0 = time.perf_counter()
            for x, P1, P2, clip, qw, sw in prepared:
                oracle.linear(x, P1, P2, clip, wl.bits_a, qw, sw, wl.group_w)
            return time.perf_counter() - t0

    ops = sum(2.0 * rows * x.shape[1] * qw.shape[0] for x, _, _, _, qw, _ in prepared)
    dt = timed_run(1)
    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
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
    sample = (f"{rows} token rows of loop 0 of each quantized input of layer 0 (q|k|v, o, up, down) at full K "
              f"and N; weight quantization and input drawing not timed; host {cpu}, numpy {np.__version__}, "
              f"BLAS {blas}")
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
    import torch

    from bit_ptq_looped_amd import loopq as lq
    from bit_ptq_looped_amd import synth

    lq.load()
    torch.cuda.set_device(0)

    if args.profile_decode:
        _, dmods = build_decode(lq, synth, torch, 1, 4)
        torch.cuda.synchronize()
        for i in range(args.profile_decode):
            decode_loop_step(lq, dmods, i % 4)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_decode} decode loop-steps", flush=True)
        return
    if args.profile_reuse:
        _, dmods = build_decode(lq, synth, torch, 1, 4)
        calibration_copy(args, torch)
        src = torch.ones(32 << 20, dtype=torch.float32, device="cuda")  # 128 MiB: more than the L2s hold
        dst = torch.empty_like(src)
        for _ in range(args.profile_reuse):
            for m in dmods:
                dst.copy_(src)
                codes, scales = m.weights[0]
                lq.loopq_looped_forward(m.x, m.P1, m.P2, m.clips, 4, codes, scales, 32, m.N, m.yT,
                                        lq.LOOPQ_SCHED_WEIGHT_STATIONARY, m.wsT)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_reuse} rounds of the decode reuse call", flush=True)
        return
    if args.profile_stack:
        _, smods = build_stack(lq, synth, torch, args.M, args.layers)
        calibration_copy(args, torch)
        for _ in range(args.profile_stack):
            stack_step(lq, smods, args.T, args.layers)
        torch.cuda.synchronize()
        print(f"profiled {args.profile_stack} stack steps (T={args.T}, {args.layers} layers)", flush=True)
        return
    if args.profile_hessian or args.profile_steps:
        wl, mods = setup_block(lq, synth, torch)
        calibration_copy(args, torch)
        if args.profile_hessian:
            hessian_setup(lq, torch, mods, wl.T, wl.M)
            for _ in range(args.profile_hessian):
                hessian_step(lq, mods)
            torch.cuda.synchronize()
            print(f"profiled {args.profile_hessian} trajectory Hessian steps", flush=True)
        else:
            run_steps(lq, mods, 4, args.profile_schedule, args.profile_steps)
            torch.cuda.synchronize()
            print(f"profiled {args.profile_steps} steps", flush=True)
        return

    if args.no_stack:
        out = {"metric": METRIC, "value": None, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "note": "headline stack skipped (--no-stack)"}
        secondary(lq, synth, torch, args, out, synth.large_prefill_workload(T=1, M=args.M, layers=args.layers))
        return
    print(f"bench: headline stack M={args.M} layers={args.layers} T={args.T}", file=sys.stderr, flush=True)
    st = stack_bench(lq, synth, torch, args)
    T, M, L = args.T, args.M, args.layers
    dt = st["dt"]
    ops_loop = st["ops_step"] / T
    out = {
        "metric": METRIC,
        "value": st["ops_step"] / dt / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights and activations (e2m3 fp6 MFMA operands), fp32 fold and accumulate",
        "data": "synthetic",
        "config": {
            "workload": st["wl"].name.replace(f"T={STACK_DRAWN_LOOPS}", f"T={T}") + f", {L} layers",
            "M": M, "T": T, "layers": L, "hidden": 2560, "intermediate": 6912,
            "linears": "q|k|v fused (2560->7680), o 2560->2560, up 2560->6912, down 6912->2560",
            "bits": "W4A4", "group_a": 32, "group_w": 32,
            "factors": "(40,64) for K=2560, (64,108) for K=6912",
            "schedule": "loop-sequential: for each loop, the layers in order, each layer's four quantized inputs "
                        "one loopq_looped_forward call over M rows (transform+quantizer, GEMM)",
            "inputs": "per input, 4 drawn loop inputs (bf16, 0.5% outlier channels x30, mean shift 0.1 t); loop t "
                      "reads input t mod 4 with its own clip; layer 0 weights packed from seeded fp32 weights, "
                      "layers 1.. seeded random packed codes and fp16 steps",
        },
        "roofline": st["roofline"],
        "ms_per_loop_step": dt * 1e3 / T,
        "tops_per_loop_step": ops_loop / (dt / T) / 1e12,
        "gbps_per_loop_step": st["bytes_loop"] / (dt / T) / 1e9,
        "frac_int8_peak": ops_loop / (dt / T) / 1e12 / INT8_PEAK_TOPS,
        "frac_hbm_peak": st["bytes_loop"] / (dt / T) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms_per_step": st["kernels_ms_per_step"],
        "fold_inclusive": st["fold_inclusive"],
        "ms_per_step_with_timing_hooks": st["ms_per_step_with_timing_hooks"],
        "t_sweep": st["t_sweep"],
        "device": torch.cuda.get_device_name(0),
    }
    stack_wl = st["wl"]
    del st
    torch.cuda.empty_cache()
    secondary(lq, synth, torch, args, out, stack_wl)


def secondary(lq, synth, torch, args, out, stack_wl):
    print("bench: secondary lines", file=sys.stderr, flush=True)

    if not args.no_block:
        wl, mods = setup_block(lq, synth, torch)
        T2, M2 = wl.T, wl.M
        out["ouro_block"] = block_bench(lq, torch, wl, mods, max(5, args.steps), max(2, args.warmup))
        if not args.no_loop_dependent:
            out["ouro_block"]["loop_dependent"] = loop_dependent_bench(lq, synth, torch, wl, mods, 5, 2)
        if not args.no_per_token:
            out["ouro_block"]["per_token"] = per_token_bench(lq, torch, mods, T2, M2, 5, 2)
        if not args.no_hessian:
            out["ouro_block"]["trajectory_hessian"] = hessian_bench(lq, torch, mods, T2, M2, 4, 2)
            out["ouro_block"]["trajectory_hessian"]["side_output"] = hessian_side_bench(lq, torch, mods, T2, M2, 4)
        del mods
        torch.cuda.empty_cache()
    if not args.no_huginn_core:
        out["huginn_core"] = huginn_core_bench(lq, synth, torch, 2)
    if not args.no_cta:
        print("bench: cta", file=sys.stderr, flush=True)
        out["cta"] = cta_bench(lq, synth, torch, 4)
    if not args.no_recurrence:
        out["recurrence"] = [recurrence_bench(lq, synth, torch, 1, 32, 20),
                             recurrence_bench(lq, synth, torch, 2048, 32, 2)]
    if not args.no_decode:
        torch.cuda.empty_cache()
        out["decode"] = [decode_bench(lq, synth, torch, Md, 4, args.decode_steps) for Md in (1, 4, 16)]
    if not args.no_cpu_baseline:
        print("bench: oracle sample on the host", file=sys.stderr, flush=True)
        cb = cpu_baseline(stack_wl, args.cpu_rows)
        out["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        out["cpu_baseline_all_cores"] = {k: cb["all_cores"][k] for k in ("value", "unit", "cores", "kind", "sample")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
