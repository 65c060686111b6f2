"""Parity at the workloads' full sizes, in the launch configuration bench.py
times: loopq_looped_forward with the default (weight-stationary) schedule over
all T*M rows of one quantized input, checked on sampled outputs the oracle
computes row by row.

* Packed weights: the exported codes and fp16 steps of the whole matrix are
  bit-exact against the oracle's weight quantization.
* Quantizer: loopq_quant_act over all T*M rows (clip of loop 0) with the x~
  dump; on sampled rows the dump is within the fp32-class bound of the
  oracle's fp64 transform (``xt_check``), and codes and steps are bit-exact
  against the oracle applied to the dump.
* y: sampled (loop, row) pairs, all N columns, against the oracle applied to
  the same x~ with the loop's clip: max|y - y_oracle| / max|y_oracle| <= 1e-4
  over the sampled rows.

Inputs are the seeded generators' full tensors, except for the Huginn-like
recurrence, whose host-side generation at 65,536 rows x K = 17,920 takes about
a minute per input: there a 256-row seeded block of the same recurrence is
repeated along M on the device.  Rows are independent in this computation, so
the launch is still the full-size one, and samples from several repeats check
every tile position against the same oracle rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from xt_check import check_xt, gpu_xt, hessian_bound

pytestmark = pytest.mark.gpu

Y_TOL = 1e-4
HUGINN_BLOCK_ROWS = 256


def say(*a):
    print(*a, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def groups_by_input(wl):
    g = {}
    for lin in wl.linears:
        g.setdefault(lin.act, []).append(lin)
    return g


def sample_rows(M, block=None):
    rows = sorted({0, 1, 31, 32, M // 2 + 5, M - 33, M - 1})
    if block:
        rows = sorted(set(rows) | {block - 1, block + 3, 3 * block + 17})
    return [r for r in rows if 0 <= r < M]


def sample_loops(T):
    return sorted({0, 1, T // 2, T - 1})


def run_case(lq, wl, act, tile_rows=None, per_loop_calls=False):
    """per_loop_calls: one loopq_looped_forward call of M rows per loop (the
    launch configuration of the headline stack), else one weight-stationary
    call over all T * M rows."""
    lins = groups_by_input(wl)[act]
    K = lins[0].K
    gw = wl.group_w
    W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
    N = W.shape[0]
    P1, P2 = synth.factors_for(wl, act, K)
    clips = synth.clips_for(wl, act)
    T, M = wl.T, wl.M
    say(f"{wl.name}: input {act} K={K} N={N} T={T} M={M} bits_a={wl.bits_a} g_w={gw}")

    # weights: GPU pack of the whole matrix vs the oracle's quantization
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(W), gw, codes, scales)
    qw, sw = oracle.quant_weights(W, gw)
    gc = torch.empty((N, K), dtype=torch.int8, device="cuda")
    gs = torch.empty((N, math.ceil(K / gw)), dtype=torch.int16, device="cuda")
    lq.loopq_export_weights(codes, scales, K, N, gw, gc, gs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gc.cpu().numpy(), qw)
    np.testing.assert_array_equal(gs.cpu().numpy().view(np.uint16), sw.view(np.uint16))
    del gc, gs

    # activations [T][M][K] on the device (bf16), and the oracle's fp32 rows
    if tile_rows:
        bits, x32 = synth.activations_for(wl, act, K, rows=tile_rows)
        x = bf16_dev(bits).repeat(1, M // tile_rows, 1).contiguous()
        src = lambda t, m: x32[t, m % tile_rows]
    else:
        bits, x32 = synth.activations_for(wl, act, K)
        x = bf16_dev(bits)
        src = lambda t, m: x32[t, m]
    del bits

    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    tP1 = dev(P1) if P1 is not None else None
    tP2 = dev(P2) if P2 is not None else None
    if per_loop_calls:
        ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, 1, M, K, N, wl.bits_a)
        for t in range(T):
            lq.loopq_looped_forward(x[t:t + 1], tP1, tP2, [clips[t]], wl.bits_a, codes, scales, gw, N, y[t:t + 1],
                                    lq.LOOPQ_SCHED_WEIGHT_STATIONARY, ws)
    else:
        ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, wl.bits_a)
        lq.loopq_looped_forward(x, tP1, tP2, clips, wl.bits_a, codes, scales, gw, N, y,
                                lq.LOOPQ_SCHED_AUTO, ws)
    torch.cuda.synchronize()
    del ws

    ts = sample_loops(T)
    ms = sample_rows(M, tile_rows)
    idx_t = torch.tensor(ts, device="cuda")
    idx_m = torch.tensor(ms, device="cuda")
    ys = y.index_select(0, idx_t).index_select(1, idx_m).cpu().numpy()  # [len(ts)][len(ms)][N]
    del y

    # quantizer over all T*M rows (loop-0 clip) with the x~ dump, sampled
    rows_all = T * M
    xf = x.view(rows_all, K)
    qc = torch.empty((rows_all, K), dtype=torch.int8, device="cuda")
    qs = torch.empty((rows_all, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((rows_all, K), dtype=torch.float32, device="cuda") if P1 is not None else None
    lq.loopq_quant_act(xf, tP1, tP2, float(clips[0]), wl.bits_a, qc, qs, xt)
    torch.cuda.synchronize()
    flat = [t * M + m for t in ts for m in ms]
    fi = torch.tensor(flat, device="cuda")
    gcodes = qc.index_select(0, fi).cpu().numpy()
    gsteps = qs.index_select(0, fi).cpu().numpy()
    xr = np.stack([src(t, m) for t in ts for m in ms])
    if xt is None:
        dump = xr.astype(np.float32)
    else:
        dump = xt.index_select(0, fi).cpu().numpy()
        ratio = check_xt(dump, xr, P1, P2)
        say(f"  x~: {dump.size} sampled elements within the fp32-class bound (max error/bound {ratio:.3f})")
    del qc, qs, xt
    qa, sa = oracle.quant_act(dump, float(clips[0]), wl.bits_a)
    np.testing.assert_array_equal(gcodes, qa)
    np.testing.assert_array_equal(gsteps.view(np.uint32), sa.view(np.uint32))

    # y of the sampled rows against the oracle applied to the same x~
    dump = dump.reshape(len(ts), len(ms), K)
    ref = np.empty(ys.shape, dtype=np.float64)
    for a, t in enumerate(ts):
        ref[a], _, _ = oracle.linear(dump[a], None, None, float(clips[t]), wl.bits_a, qw, sw, gw)
    err = float(np.max(np.abs(ys - ref)) / np.max(np.abs(ref)))
    say(f"  y: {len(ts)} loops x {len(ms)} rows x {N} columns, rel err {err:.3e}")
    assert err <= Y_TOL


OURO_INPUTS = ["qkv_in", "o_in", "up_in", "down_in"]


@pytest.mark.parametrize("bits_a", [4, 8])
@pytest.mark.parametrize("act", OURO_INPUTS)
def test_fullsize_ouro_block(lq, act, bits_a):
    run_case(lq, synth.ouro_block_workload(bits_a=bits_a), act)


@pytest.mark.parametrize("act", ["adapter_in", "core_in", "proj_in"])
def test_fullsize_huginn(lq, act):
    run_case(lq, synth.huginn_workload(), act, tile_rows=HUGINN_BLOCK_ROWS)


@pytest.mark.parametrize("act", OURO_INPUTS)
def test_fullsize_large_prefill(lq, act):
    run_case(lq, synth.large_prefill_workload(T=4), act)


@pytest.mark.parametrize("act", OURO_INPUTS)
def test_fullsize_large_prefill_per_loop_calls(lq, act):
    """The headline stack's launch configuration: one call of M = 8192 rows
    per loop (transform + quantizer launch, GEMM launch)."""
    run_case(lq, synth.large_prefill_workload(T=4), act, per_loop_calls=True)


@pytest.mark.parametrize("act", ["qkv_in", "down_in"])
def test_fullsize_large_prefill_T8(lq, act):
    """T = 8: all 65,536 rows of an input in one weight-stationary launch."""
    run_case(lq, synth.large_prefill_workload(T=8), act)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("act", OURO_INPUTS)
def test_fullsize_decode(lq, act, M):
    """Decode calls at the block's full N and K (the bench's decode stack), both
    schedules: loop by loop (M rows per launch) and weight-stationary (T*M
    rows per launch, where they fit the few-row kernel).  Every row and column
    against the oracle applied to the kernel's x~."""
    wl = synth.ouro_block_workload(bits_a=4, M=M, T=4)
    lins = groups_by_input(wl)[act]
    K = lins[0].K
    W = np.concatenate([synth.weights_for(wl, lin) for lin in lins], axis=0)
    N = W.shape[0]
    P1, P2 = synth.factors_for(wl, act, K)
    clips = synth.clips_for(wl, act)
    T = wl.T
    say(f"decode {act} K={K} N={N} M={M} T={T}")
    codes, scales = lq.empty_packed_weights(K, N, 32)
    lq.loopq_pack_weights(dev(W), 32, codes, scales)
    qw, sw = oracle.quant_weights(W, 32)
    bits, x32 = synth.activations_for(wl, act, K)
    x = bf16_dev(bits)
    xt = gpu_xt(lq, x.view(T * M, K), x32.reshape(T * M, K), P1, P2).reshape(T, M, K)
    ref = oracle.looped_forward(xt, None, None, clips, 4, qw, sw, 32)
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4)
    for schedule in (1, 2):
        y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
        lq.loopq_looped_forward(x, dev(P1), dev(P2), clips, 4, codes, scales, 32, N, y, schedule, ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        say(f"  schedule {schedule}: rel err {err:.3e}")
        assert err <= Y_TOL


# ---------------------------------------------------------------------------
# the NEXT rows at the bench's sizes
# ---------------------------------------------------------------------------

def sample_pairs(K, n, key):
    """n (i, j) pairs of H: the corners and diagonal, tile edges, and seeded
    random pairs (both triangles)."""
    rng = synth.seeded_rng(synth.TEST, 220, K, key)
    fixed = [(0, 0), (K - 1, K - 1), (0, K - 1), (K - 1, 0), (127, 128), (128, 127), (K // 2, K // 2 + 1)]
    return fixed + [tuple(int(v) for v in rng.integers(0, K, size=2)) for _ in range(n)]


@pytest.mark.parametrize("act", ["qkv_in", "down_in"])
def test_fullsize_trajectory_hessian(lq, act):
    """The bench's trajectory Hessian: the x~ of all T*M = 4096 rows of one
    block input (the quantizer's dump) accumulated in one call; sampled
    elements against the fp64 sum over the rows, computed one by one, within
    the bound of the kernel's plane-product arithmetic (xt_check.hessian_bound);
    exact symmetry."""
    wl = synth.ouro_block_workload()
    K = groups_by_input(wl)[act][0].K
    P1, P2 = synth.factors_for(wl, act, K)
    bits, x32 = synth.activations_for(wl, act, K)
    rows = wl.T * wl.M
    say(f"hessian {act} rows={rows} K={K}")
    xdev = bf16_dev(bits.reshape(rows, K))
    codes = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    steps = torch.empty((rows, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    lq.loopq_quant_act(xdev, dev(P1), dev(P2), 1.0, 4, codes, steps, xt)
    H = torch.zeros((K, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_HESSIAN, 0, rows, K, 0, 0), dtype=torch.uint8,
                     device="cuda")
    lq.loopq_hessian_accumulate(xt, H, ws)
    torch.cuda.synchronize()
    X = xt.cpu().numpy().astype(np.float64)
    check_xt(X[sample_rows(rows)].astype(np.float32), x32.reshape(rows, K)[sample_rows(rows)], P1, P2)
    Hc = H.cpu().numpy()
    assert np.array_equal(Hc, Hc.T)
    worst = 0.0
    for i, j in sample_pairs(K, 400, 1):
        want = float(X[:, i] @ X[:, j])
        mag = float(np.abs(X[:, i]) @ np.abs(X[:, j]))
        bound = hessian_bound(rows, mag)
        err = abs(float(Hc[i, j]) - want)
        assert err <= bound, (i, j, err, bound)
        worst = max(worst, err / max(bound, 1e-300))
    say(f"  max error / bound {worst:.3g}")


def test_fullsize_per_token_loop(lq):
    """The bench's per-token step for the up input (K = 2048, N = 5632, T = 4,
    M = 1024) in one loopq_looped_forward_per_token call; sampled (loop, row)
    pairs against the oracle's per-token linear on the kernel's x~."""
    wl = synth.ouro_block_workload()
    act = "up_in"
    lins = groups_by_input(wl)[act]
    K, N = lins[0].K, sum(l.N for l in lins)
    T, M = wl.T, wl.M
    P1, P2 = synth.factors_for(wl, act, K)
    bits, x32 = synth.activations_for(wl, act, K)
    clips = [float(c) for c in synth.clips_for(wl, act)]
    W = np.concatenate([synth.weights_for(wl, l) for l in lins], axis=0)
    codes, scales = lq.empty_packed_weights(K, N, wl.group_w)
    lq.loopq_pack_weights(dev(W), wl.group_w, codes, scales)
    xdev = bf16_dev(bits)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, 4),
                     dtype=torch.uint8, device="cuda")
    say(f"per-token loop {act} T={T} M={M} K={K} N={N}")
    lq.loopq_looped_forward_per_token(xdev, dev(P1), dev(P2), clips, 4, codes, scales, wl.group_w, N, y, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(W, wl.group_w)
    got = y.cpu().numpy()
    rows = sample_rows(M)
    for t in sample_loops(T):
        xt = gpu_xt(lq, bf16_dev(bits[t][rows]), x32[t][rows], P1, P2)
        ref, _, _ = oracle.linear_per_token(xt, None, None, clips[t], 4, qw, sw, wl.group_w)
        err = float(np.max(np.abs(got[t][rows] - ref)) / np.max(np.abs(ref)))
        say(f"  loop {t}: rel err {err:.2e}")
        assert err <= Y_TOL


def test_fullsize_adapter_recurrence_decode(lq):
    """The bench's Huginn-like adapter loop at M = 1: adapter 10560 -> 5280,
    weight groups of 128, A8, T = 32 dependent loops in one call; every loop
    against the oracle's linear on cat(s_t, e) with the GPU's own state."""
    N, K, gw, T = 5280, 10560, 128, 32
    rng = synth.seeded_rng(synth.HUGINN, synth.T_W, 99)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.5 / np.sqrt(K))
    s0 = synth.seeded_rng(synth.HUGINN, synth.T_X, 99).standard_normal((1, N), dtype=np.float32)
    e = synth.seeded_rng(synth.HUGINN, synth.T_AUX, 99).standard_normal((1, N), dtype=np.float32)
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(w), gw, codes, scales)
    y = torch.empty((T, 1, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, 1, 0, N, 8), dtype=torch.uint8,
                     device="cuda")
    say(f"adapter recurrence M=1 T={T} N={N} K={K}")
    lq.loopq_recurrent_adapter(dev(s0), dev(e), None, None, [1.0] * T, 8, codes, scales, gw, y, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(w, gw)
    got = y.cpu().numpy()
    worst = 0.0
    for t in range(T):
        state = s0 if t == 0 else got[t - 1]
        x = np.concatenate([state, e], axis=1).astype(np.float32)
        ref, _, _ = oracle.linear(x, None, None, 1.0, 8, qw, sw, gw)
        err = float(np.max(np.abs(got[t] - ref)) / np.max(np.abs(ref)))
        worst = max(worst, err)
        assert err <= Y_TOL, (t, err)
    say(f"  worst loop rel err {worst:.2e}, final max|s| {np.max(np.abs(got[-1])):.3g}")
