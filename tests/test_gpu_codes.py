"""The activation codes the product actually consumes, bit for bit.

Every forward path keeps its codes in the form its product reads: e2m3 fp6
MFMA operands (W4A4 GEMM), int8 tiles (W4A8 GEMM), or LDS (few-row kernel,
which also writes them to the workspace).  ``loopq_export_act_codes`` turns
what a forward call left in its workspace back into canonical codes and
steps; this module compares them with Eq.(4) ("paper_specification.yaml",
lq1_quantization) applied by the oracle to the kernel's own x~ (the
``xt_out`` dump of ``loopq_quant_act`` for the same rows), bit for bit.
That also pins the reading that every entry point quantizes the same x~ for
the same rows.

Against the oracle's fp64 transform the codes may differ only at near-ties:
where the exact quotient x~64 / s64 lies within the propagated fp32-class
transform error of a rounding boundary (``test_codes_vs_fp64_transform``).
"""

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from xt_check import check_xt, xt_bound

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(*a):
    print(*a, flush=True)


def pack(lq, w32, gw):
    N, K = w32.shape
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(w32), gw, codes, scales)
    return codes, scales


def inputs(T, M, K, dtype, key, zero_rows=(), hot=None):
    """[T][M][K] activations (device tensor, fp32 host copy) with outlier
    channels, some all-zero rows and optionally one huge element per row."""
    x = synth.with_outliers(synth.gaussian((T, M, K), 300, key, T, M, K), max(1, K // 100), 20.0, 301, key)
    if hot is not None:
        x[:, :, hot] = 500.0
    for t, m in zero_rows:
        x[t, m] = 0.0
    if dtype == "bf16":
        bits16, x32 = synth.round_to_bf16(x)
        return torch.from_numpy(bits16.view(np.int16)).cuda().view(torch.bfloat16), x32
    return dev(x), x


def kernel_xt(lq, xdev, x32, P1, P2):
    """The kernel's x~ of these rows (rows x K fp32), bound-checked; x itself
    without a transform."""
    rows, K = x32.shape
    if P1 is None:
        return x32
    c = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    s = torch.empty((rows, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    lq.loopq_quant_act(xdev.reshape(rows, K), dev(P1), dev(P2), 1.0, 4, c, s, xt)
    torch.cuda.synchronize()
    dump = xt.cpu().numpy()
    check_xt(dump, x32, P1, P2)
    return dump


def export(lq, ws, op, T, M, K, N, bits, schedule):
    rows = T * M
    c = torch.full((rows, K), 99, dtype=torch.int8, device="cuda")
    s = torch.full((rows, K // 32), -1.0, dtype=torch.float32, device="cuda")
    lq.loopq_export_act_codes(ws, op, T, M, K, N, bits, schedule, c, s)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def oracle_codes(xt, T, M, clips, bits, per_token=False):
    K = xt.shape[1]
    cs, ss = [], []
    for t in range(T):
        q, s = oracle.quant_act(np.ascontiguousarray(xt[t * M:(t + 1) * M]), float(clips[t]), bits,
                                group=K if per_token else 32)
        if per_token:
            s = np.repeat(s, K // 32, axis=1)
        cs.append(q.astype(np.int8))
        ss.append(s)
    return np.concatenate(cs), np.concatenate(ss)


def assert_codes_equal(got_c, got_s, want_c, want_s, what):
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[:3].tolist()}"
    np.testing.assert_array_equal(got_s.view(np.uint32), want_s.view(np.uint32), err_msg=what)


# (name, T, M, K, factors, bits, schedule, dtype, N, clip scale, zero rows, hot column)
CASES = [
    # the GEMM paths at the block shapes: fp6 operands (A4) and int8 tiles (A8)
    ("block qkv_in A4 weight-stationary", 4, 1024, 2048, (32, 64), 4, 2, "bf16", 256, 1.0, [(0, 5), (3, 1023)], None),
    ("block down_in A4 weight-stationary", 4, 256, 5632, (64, 88), 4, 2, "bf16", 64, 1.0, [(1, 0)], None),
    ("block qkv_in A8 weight-stationary", 4, 512, 2048, (32, 64), 8, 2, "bf16", 128, 1.0, [(2, 7)], None),
    ("2.6B-like down_in A4", 2, 128, 6912, (64, 108), 4, 2, "bf16", 64, 1.0, [], None),
    ("2.6B-like qkv_in A4 loop-sequential", 3, 96, 2560, (40, 64), 4, 1, "bf16", 64, 1.0, [], None),
    # ragged rows per loop, loop-sequential (one tiled buffer per loop)
    ("ragged loop-sequential A4", 3, 100, 2048, (32, 64), 4, 1, "f32", 96, 1.0, [(1, 99)], None),
    ("ragged loop-sequential A8", 3, 100, 2048, (32, 64), 8, 1, "f32", 96, 1.0, [], None),
    # an odd number of groups (the last fp6 pair half empty), generic factor shape
    ("odd groups, factors (12, 24)", 2, 40, 288, (12, 24), 4, 2, "f32", 40, 1.0, [(0, 0)], None),
    # no transform: the plain quantizer's fp6 path (8 lanes per group, software e2m3)
    ("no transform, odd groups A4", 2, 70, 96, None, 4, 2, "f32", 40, 1.0, [(1, 3)], None),
    ("no transform A8", 2, 70, 160, None, 8, 2, "bf16", 40, 1.0, [], None),
    # saturation: small clips and one huge element per row
    ("saturated groups A4", 2, 64, 256, (16, 16), 4, 2, "f32", 64, 0.3, [(0, 1)], 17),
    ("saturated groups A8, no transform", 2, 64, 256, None, 8, 2, "f32", 64, 0.3, [], 40),
    # the few-row kernel (at most 16 rows per launch)
    ("few-row, transform in the launch (T*M = 4)", 4, 1, 2048, (32, 64), 4, 2, "bf16", 2048, 1.0, [], None),
    ("few-row loop-sequential (64, 88)", 4, 1, 5632, (64, 88), 4, 1, "bf16", 96, 1.0, [], None),
    ("few-row three-launch form (16 rows)", 1, 16, 2048, (32, 64), 4, 2, "bf16", 64, 1.0, [(0, 3)], None),
    ("few-row MFMA form, 12 rows", 3, 4, 2048, (32, 64), 8, 2, "bf16", 64, 1.0, [], None),
    ("few-row, no transform, K = 10560, A8", 2, 2, 10560, None, 8, 2, "f32", 64, 1.0, [(1, 1)], None),
    # fp32 inputs of the few-row kernel (the fp32 transform path)
    ("few-row fp32, (16, 16), 16 rows", 1, 16, 256, (16, 16), 4, 2, "f32", 128, 1.0, [(0, 2)], None),
    ("few-row fp32, (16, 16), 4 rows", 1, 4, 256, (16, 16), 4, 2, "f32", 128, 1.0, [], None),
    ("few-row fp32, (32, 64), 2 rows", 2, 1, 2048, (32, 64), 4, 2, "f32", 64, 1.0, [], None),
    ("few-row fp32 loop-sequential (16, 16)", 4, 16, 256, (16, 16), 4, 1, "f32", 128, 1.0, [], None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_codes_are_eq4_of_the_kernel_xt(lq, case):
    name, T, M, K, fac, bits, sched, dtype, N, cscale, zero_rows, hot = case
    say(f"forward codes: {name}: T={T} M={M} K={K} factors={fac} A{bits} schedule={sched}")
    rng = synth.seeded_rng(synth.TEST, 310, K, M, T)
    P1 = P2 = None
    if fac is not None:
        P1, P2 = synth.haar_orthogonal(fac[0], rng), synth.haar_orthogonal(fac[1], rng)
    xdev, x32 = inputs(T, M, K, dtype, K + M, zero_rows, hot)
    clips = (synth.uniform((T,), 0.6, 1.0, 311, K) * np.float32(cscale)).astype(np.float32)
    w = synth.gaussian((N, K), 312, K, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits)
    lq.loopq_looped_forward(xdev, None if P1 is None else dev(P1), None if P2 is None else dev(P2), clips, bits,
                            codes, scales, 32, N, y, sched, ws)
    torch.cuda.synchronize()
    gc, gs = export(lq, ws, lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits, sched)
    xt = kernel_xt(lq, xdev, x32.reshape(T * M, K), P1, P2)
    wc, wsx = oracle_codes(xt, T, M, clips, bits)
    assert_codes_equal(gc, gs, wc, wsx, name)
    for t, m in zero_rows:
        r = t * M + m
        assert np.all(gc[r] == 0) and np.all(gs[r] == 0)
    if hot is not None and P1 is None:  # untransformed: the huge element saturates its code
        assert np.all(np.abs(gc[:, hot]) == oracle.qmax_for_bits(bits))
    # and the product is the oracle's product of these codes (sampled rows:
    # the first, a middle and the last row of every loop)
    qw, sw = oracle.quant_weights(w, 32)
    rows = sorted({t * M + m for t in range(T) for m in (0, M // 2, M - 1)})
    ref = oracle.rescale_dots(wsx[rows], oracle.group_dots(wc[rows], qw), sw, 32)
    got = y.cpu().numpy().reshape(T * M, N)[rows].astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-4 * max(np.max(np.abs(ref)), 1e-30)


@pytest.mark.parametrize("T,M,K,fac,bits", [(2, 64, 2048, (32, 64), 4), (2, 3, 2048, (32, 64), 4),
                                            (2, 48, 256, None, 4), (1, 40, 2048, (32, 64), 8)])
def test_per_token_forward_codes(lq, T, M, K, fac, bits):
    say(f"per-token forward codes T={T} M={M} K={K} factors={fac} A{bits}")
    rng = synth.seeded_rng(synth.TEST, 320, K, M)
    P1 = P2 = None
    if fac is not None:
        P1, P2 = synth.haar_orthogonal(fac[0], rng), synth.haar_orthogonal(fac[1], rng)
    xdev, x32 = inputs(T, M, K, "bf16", 321 + M, [(0, 1)])
    clips = synth.uniform((T,), 0.6, 1.0, 322, K)
    N = 64
    w = synth.gaussian((N, K), 323, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, bits)
    lq.loopq_looped_forward_per_token(xdev, None if P1 is None else dev(P1), None if P2 is None else dev(P2), clips,
                                      bits, codes, scales, 32, N, y, ws)
    torch.cuda.synchronize()
    gc, gs = export(lq, ws, lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, bits, 0)
    xt = kernel_xt(lq, xdev, x32.reshape(T * M, K), P1, P2)
    wc, wsx = oracle_codes(xt, T, M, clips, bits, per_token=True)
    assert_codes_equal(gc, gs, wc, wsx, "per-token forward")


def test_recurrent_adapter_last_loop_codes(lq):
    M, N, T, bits = 3, 48, 3, 8
    say(f"recurrent adapter codes M={M} N={N} T={T}")
    s0 = synth.gaussian((M, N), 330)
    e = synth.gaussian((M, N), 331)
    w = synth.gaussian((N, 2 * N), 332, scale=0.1)
    codes, scales = pack(lq, w, 32)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, M, 0, N, bits)
    clips = [0.9, 0.8, 0.7]
    lq.loopq_recurrent_adapter(dev(s0), dev(e), None, None, clips, bits, codes, scales, 32, y, ws)
    torch.cuda.synchronize()
    gc, gs = export(lq, ws, lq.LOOPQ_OP_RECURRENT_ADAPTER, 1, M, 2 * N, N, bits, 0)
    state = y.cpu().numpy()[T - 2]
    x_last = np.concatenate([state, e], axis=1).astype(np.float32)
    wc, wsx = oracle.quant_act(x_last, clips[T - 1], bits)
    assert_codes_equal(gc, gs, wc.astype(np.int8), wsx, "adapter, last loop")


# ------------------------------------------------------------- vs the fp64 transform

def near_tie_check(codes, steps, x32, P1, P2, clips_rows, bits):
    """Codes of the kernel against Eq.(4) of the oracle's fp64 transform: a
    difference is allowed only where the exact quotient x~64 / s64 lies within
    the propagated transform error of a rounding boundary (k + 1/2), and then
    by one.  Steps agree within the same relative error.  Returns the number
    of differing codes."""
    qmax = oracle.qmax_for_bits(bits)
    rows, K = x32.shape
    x64 = oracle.kron_transform(x32, P1, P2)
    b = xt_bound(x32, P1, P2)
    G = K // 32
    xg = x64.reshape(rows, G, 32)
    bg = b.reshape(rows, G, 32)
    amax = np.max(np.abs(xg), axis=2)
    bA = np.max(bg, axis=2)
    c = np.asarray(clips_rows, dtype=np.float64)[:, None]
    s64 = c * amax / qmax
    rel_s = np.where(amax > 0, bA / np.where(amax > 0, amax, 1.0), 0.0) + 2.0 ** -22
    s32 = steps.astype(np.float64)
    assert np.all(np.abs(s32 - s64) <= s64 * rel_s * 1.01 + 1e-300), "steps outside the transform error"
    safe = np.where(s64 > 0, s64, 1.0)[:, :, None]
    q64 = xg / safe
    want = np.clip(np.rint(q64), -qmax, qmax)
    want[(s64 == 0)] = 0
    tol = bg / safe * 1.01 + np.abs(q64) * (rel_s[:, :, None] * 1.01 + 2.0 ** -23) + 2.0 ** -20
    got = codes.reshape(rows, G, 32).astype(np.float64)
    diff = got != want
    if np.any(diff):
        dist = np.abs(np.abs(q64 - np.floor(q64)) - 0.5)  # distance to the nearest k + 1/2
        ok = (np.abs(got - want) == 1) & (dist <= tol)
        bad = diff & ~ok
        assert not np.any(bad), (f"{np.count_nonzero(bad)} codes differ from the fp64 transform's away from a "
                                 f"near-tie; first {np.argwhere(bad)[:3].tolist()}")
    return int(np.count_nonzero(diff))


@pytest.mark.parametrize("fac,T,M,bits,sched", [((32, 64), 4, 1024, 4, 2), ((64, 88), 4, 256, 4, 2),
                                                ((32, 64), 2, 512, 8, 2), ((40, 64), 2, 256, 4, 1),
                                                ((64, 108), 2, 64, 4, 2), ((32, 64), 4, 1, 4, 2),
                                                ((64, 88), 4, 1, 4, 1)])
def test_codes_vs_fp64_transform_differ_only_at_near_ties(lq, fac, T, M, bits, sched):
    K = fac[0] * fac[1]
    say(f"near-tie check factors={fac} T={T} M={M} A{bits} schedule={sched}")
    rng = synth.seeded_rng(synth.TEST, 340, K, M)
    P1, P2 = synth.haar_orthogonal(fac[0], rng), synth.haar_orthogonal(fac[1], rng)
    xdev, x32 = inputs(T, M, K, "bf16", 341 + M)
    clips = synth.uniform((T,), 0.6, 1.0, 342, K)
    N = 64
    codes, scales = pack(lq, synth.gaussian((N, K), 343, scale=0.02), 32)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits)
    lq.loopq_looped_forward(xdev, dev(P1), dev(P2), clips, bits, codes, scales, 32, N, y, sched, ws)
    torch.cuda.synchronize()
    gc, gs = export(lq, ws, lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, bits, sched)
    clips_rows = np.repeat(np.asarray(clips, dtype=np.float64), M)
    n = near_tie_check(gc, gs, x32.reshape(T * M, K), P1, P2, clips_rows, bits)
    say(f"  {n} of {gc.size} codes differ from the fp64 transform's, all at near-ties")
