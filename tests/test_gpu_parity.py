"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: weight codes and fp16 steps, activation codes and fp32 steps, and the
int32 group dots are bit-exact; fp32 outputs satisfy
max|y - y_oracle| / max|y_oracle| <= 1e-4.  Inputs come from the seeded
generators.  With a transform, the kernel's x~ is first checked against the
oracle's fp64 transform within the fp32-class bound of ``xt_check``; codes,
steps and y are then compared with the oracle applied to that x~ (the pages
fix no precision for the transform).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from xt_check import check_xt, gpu_xt

pytestmark = pytest.mark.gpu

Y_TOL = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def say(*a):
    print(*a, flush=True)


def pack(lq, w32, gw):
    N, K = w32.shape
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(w32), gw, codes, scales)
    return codes, scales


def export(lq, codes, scales, K, N, gw):
    c = torch.empty((N, K), dtype=torch.int8, device="cuda")
    s = torch.empty((N, math.ceil(K / gw)), dtype=torch.int16, device="cuda")
    lq.loopq_export_weights(codes, scales, K, N, gw, c, s)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy().view(np.float16)


def rel_err(y, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(y, dtype=np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def special_weights(N, K, key):
    w = synth.gaussian((N, K), key, scale=0.02)
    w[0, :32] = 0.0                          # an all-zero group
    if N > 1:
        w[1, 5] = 0.3                        # an outlier inside a group
    return w


# ------------------------------------------------------------------------ weights

@pytest.mark.parametrize("K,N,gw", [(256, 128, 32), (2048, 40, 32), (96, 33, 32), (160, 64, 128),
                                    (320, 72, 128), (10560, 8, 128)])
def test_pack_matches_oracle(lq, K, N, gw):
    say(f"pack K={K} N={N} gw={gw}")
    w = special_weights(N, K, K + N + gw)
    codes, scales = pack(lq, w, gw)
    gc, gs = export(lq, codes, scales, K, N, gw)
    oc, os_ = oracle.quant_weights(w, gw)
    np.testing.assert_array_equal(gc, oc)
    np.testing.assert_array_equal(gs.view(np.uint16), os_.view(np.uint16))


def test_pack_rejects_fp16_overflow(lq):
    w = np.zeros((4, 64), dtype=np.float32)
    w[2, 40] = 7 * 65520.0
    with pytest.raises(lq.LoopQError) as e:
        pack(lq, w, 32)
    assert e.value.status == lq.LOOPQ_ERR_RANGE


# ------------------------------------------------------------------------ activations

def _quant_gpu(lq, xdev, P1, P2, clip, bits, with_xt=False):
    M, K = xdev.shape
    codes = torch.empty((M, K), dtype=torch.int8, device="cuda")
    scales = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((M, K), dtype=torch.float32, device="cuda") if with_xt else None
    lq.loopq_quant_act(xdev, None if P1 is None else dev(P1), None if P2 is None else dev(P2),
                       clip, bits, codes, scales, xt)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (xt.cpu().numpy() if with_xt else None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K", [(1, 32), (7, 256), (33, 2048), (5, 5632)])
def test_quant_plain_matches_oracle(lq, dtype, bits, M, K):
    say(f"quant plain {dtype} A{bits} M={M} K={K}")
    x = synth.with_outliers(synth.gaussian((M, K), M, K, bits), max(1, K // 100), 20.0, K, M)
    x[0, :32] = 0.0  # zero group
    clip = float(synth.uniform((1,), 0.6, 1.0, M, K)[0])
    if dtype == "bf16":
        bits16, x32 = synth.round_to_bf16(x)
        xd = bf16_dev(bits16)
    else:
        x32, xd = x, dev(x)
    gc, gs, _ = _quant_gpu(lq, xd, None, None, clip, bits)
    oc, os_ = oracle.quant_act(x32, clip, bits)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gc, oc)


@pytest.mark.parametrize("n1,n2", [(16, 16), (32, 64), (64, 88), (40, 64), (64, 108), (4, 8)])
@pytest.mark.parametrize("dtype,bits", [("f32", 4), ("bf16", 4), ("bf16", 8)])
def test_quant_transform_matches_oracle(lq, n1, n2, dtype, bits):
    K = n1 * n2
    M = 5
    say(f"quant transform n1={n1} n2={n2} {dtype} A{bits}")
    rng = synth.seeded_rng(synth.TEST, 100, n1, n2)
    P1 = synth.haar_orthogonal(n1, rng)
    P2 = synth.haar_orthogonal(n2, rng)
    x = synth.with_outliers(synth.gaussian((M, K), 101, n1, n2), max(1, K // 100), 20.0, 102, n1)
    if dtype == "bf16":
        bits16, x32 = synth.round_to_bf16(x)
        xd = bf16_dev(bits16)
    else:
        x32, xd = x, dev(x)
    clip = 0.83
    gc, gs, gxt = _quant_gpu(lq, xd, P1, P2, clip, bits, with_xt=True)
    ratio = check_xt(gxt, x32, P1, P2)
    oc, os_ = oracle.quant_act(gxt, clip, bits)
    np.testing.assert_array_equal(gs.view(np.uint32), os_.view(np.uint32))
    np.testing.assert_array_equal(gc, oc)
    # informational: codes of the oracle's own fp64-then-rounded x~
    rc, _ = oracle.quant_act(oracle.transformed_f32(x32, P1, P2), clip, bits)
    say(f"  x~ error / bound <= {ratio:.3f}; {np.count_nonzero(rc != gc)} codes differ from the "
        f"fp64 transform's")


def test_quant_zero_rows_and_tiny_clip(lq):
    x = synth.gaussian((3, 256), 103)
    x[1] = 0.0
    gc, gs, _ = _quant_gpu(lq, dev(x), None, None, 1e-30, 4)
    oc, os_ = oracle.quant_act(x, 1e-30, 4)
    np.testing.assert_array_equal(gs, os_)
    np.testing.assert_array_equal(gc, oc)
    assert np.all(gs[1] == 0) and np.all(gc[1] == 0)


# ------------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N,gw", [(16, 256, 128, 32), (37, 512, 200, 32), (130, 2048, 96, 32),
                                      (5, 160, 64, 128), (64, 10560, 64, 128), (9, 96, 40, 32),
                                      (3, 32, 33, 32)])
def test_group_dots_bit_exact(lq, bits, M, K, N, gw):
    say(f"group dots A{bits} M={M} K={K} N={N} gw={gw}")
    qmax = oracle.qmax_for_bits(bits)
    qa = synth.seeded_rng(synth.TEST, 110, M, K, bits).integers(-qmax, qmax + 1, size=(M, K)).astype(np.int8)
    w = synth.gaussian((N, K), 111, N, K, scale=0.02)
    codes, _scales = pack(lq, w, gw)
    qw, _ = oracle.quant_weights(w, gw)
    dots = torch.empty((M, N, K // 32), dtype=torch.int32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, bits)
    lq.loopq_group_dots(dev(qa), codes, N, dots, ws, bits_a=bits)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dots.cpu().numpy().astype(np.int64), oracle.group_dots(qa, qw))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K,N,gw", [(16, 256, 128, 32), (200, 1024, 300, 32), (3, 320, 40, 128),
                                      (33, 96, 72, 32)])
def test_gemm_codes_matches_oracle(lq, bits, M, K, N, gw):
    say(f"gemm codes A{bits} M={M} K={K} N={N} gw={gw}")
    rng = synth.seeded_rng(synth.TEST, 120, M, K, N)
    qmax = oracle.qmax_for_bits(bits)
    qa = rng.integers(-qmax, qmax + 1, size=(M, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, size=(M, K // 32)).astype(np.float32)
    sa[0, 0] = 0.0
    w = synth.gaussian((N, K), 121, M, K, scale=0.02)
    codes, scales = pack(lq, w, gw)
    qw, sw = oracle.quant_weights(w, gw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, bits)
    lq.loopq_gemm_codes(dev(qa), dev(sa), codes, scales, gw, N, y, ws, bits_a=bits)
    torch.cuda.synchronize()
    ref = oracle.rescale_dots(sa, oracle.group_dots(qa, qw), sw, gw)
    assert rel_err(y.cpu().numpy(), ref) <= Y_TOL


@pytest.mark.parametrize("M,K,N,bits,gw", [(1024, 2048, 2048, 4, 32), (1000, 2080, 2000, 4, 32), (1024, 2048, 6144, 4, 32),
                                            (1024, 5632, 2048, 4, 32), (8192, 6912, 2560, 4, 32),
                                            (1024, 2048, 2048, 8, 32), (1000, 2080, 2000, 8, 32), (4096, 2048, 5632, 8, 32),
                                            (2048, 10560, 5280, 8, 128), (1000, 10528, 2000, 8, 128)],
                         ids=["four-way", "four-way ragged, odd groups", "two-way", "four-way long K",
                              "two-way, the stack's down projection",
                              "A8 four-way", "A8 four-way ragged, odd groups", "A8 two-way",
                              "A8 four-way g128, the adapter recurrence", "A8 four-way g128 ragged, short tail"])
def test_gemm_split_forms_match_oracle(lq, M, K, N, bits, gw):
    """The launch sizes at which the GEMMs take their split-K forms (two-way: 64x128 tiles over
    half of K per wave; four-way: 64x64 tiles over a quarter of K per wave, the partial sums added
    through LDS): the W4A4 kernel on fp6 operands and the W4A8 kernel on int8 operands, against
    the oracle's per-group rescale on sampled rows and columns that cover the first, last and
    tile-boundary rows and columns (the oracle's dots for the whole output would take minutes)."""
    say(f"gemm split forms M={M} K={K} N={N} A{bits} g_w={gw}")
    qmax = 7 if bits == 4 else 127
    rng = synth.seeded_rng(synth.TEST, 125, M, K, N)
    qa = rng.integers(-qmax, qmax + 1, size=(M, K)).astype(np.int8)
    sa = rng.uniform(0.01, 2.0, size=(M, K // 32)).astype(np.float32)
    w = synth.gaussian((N, K), 126, M, K, scale=0.02)
    codes, scales = pack(lq, w, gw)
    qw, sw = oracle.quant_weights(w, gw)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, bits)
    lq.loopq_gemm_codes(dev(qa), dev(sa), codes, scales, gw, N, y, ws, bits_a=bits)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    rows = sorted({0, 1, 31, 32, 63, 64, 127, 128, M // 2, M - 65, M - 64, M - 1} | set(rng.integers(0, M, 8).tolist()))
    cols = sorted({0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 65, N - 64, N - 1} | set(rng.integers(0, N, 8).tolist()))
    ref = oracle.rescale_dots(sa[rows], oracle.group_dots(qa[rows], qw[cols]), sw[cols], gw)
    assert rel_err(got[np.ix_(rows, cols)], ref) <= Y_TOL
    assert np.all(np.isfinite(got))


# ------------------------------------------------------------------------ end to end

def _tiny_gpu_and_oracle(lq, schedule):
    wl = synth.tiny_workload()
    lin = wl.linears[0]
    P1, P2 = synth.factors_for(wl, "x", lin.K)
    W = synth.weights_for(wl, lin)
    xs, _ = synth.activations_for(wl, "x", lin.K)
    clips = synth.clips_for(wl, "x")
    # GPU: fold -> pack -> looped forward, all on the device
    wf = torch.empty((lin.N, lin.K), dtype=torch.float32, device="cuda")
    fws = lq.empty_workspace(lq.LOOPQ_OP_FOLD, 0, 16, lin.K, 16, 0)
    lq.loopq_fold_weights(dev(W), dev(P1), dev(P2), wf, fws)
    codes, scales = lq.empty_packed_weights(lin.K, lin.N, 32)
    lq.loopq_pack_weights(wf, 32, codes, scales)
    y = torch.empty((wl.T, wl.M, lin.N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, wl.T, wl.M, lin.K, lin.N, 4)
    lq.loopq_looped_forward(dev(xs), dev(P1), dev(P2), clips, 4, codes, scales, 32, lin.N, y,
                            schedule, ws)
    torch.cuda.synchronize()
    # oracle: its own fold, weight quantization and loop, on the kernel's x~
    wt = oracle.fold_weights(W, P1, P2).astype(np.float32)
    qw, sw = oracle.quant_weights(wt, 32)
    T, M, K = xs.shape
    xt = gpu_xt(lq, dev(xs).view(T * M, K), xs.reshape(T * M, K), P1, P2).reshape(T, M, K)
    ref = oracle.looped_forward(xt, None, None, clips, 4, qw, sw, 32)
    return y.cpu().numpy(), ref, (codes, scales, qw, sw, lin)


@pytest.mark.parametrize("schedule", [1, 2])
def test_tiny_looped_end_to_end(lq, schedule):
    say(f"tiny looped schedule={schedule}")
    y, ref, (codes, scales, qw, sw, lin) = _tiny_gpu_and_oracle(lq, schedule)
    gc, gs = export(lq, codes, scales, lin.K, lin.N, 32)
    np.testing.assert_array_equal(gc, qw)
    np.testing.assert_array_equal(gs.view(np.uint16), sw.view(np.uint16))
    assert rel_err(y, ref) <= Y_TOL
    for t in range(ref.shape[0]):
        assert rel_err(y[t], ref[t]) <= Y_TOL


def test_schedules_agree_and_are_deterministic(lq):
    # tiny workload, M = 16, T = 4: the loop-sequential schedule launches 16
    # rows per loop (small-row kernel), the weight-stationary one 64 rows
    # (MFMA GEMM); same codes, y equal up to fp32 summation order
    y1, _, _ = _tiny_gpu_and_oracle(lq, 1)
    y1b, _, _ = _tiny_gpu_and_oracle(lq, 1)
    y2, _, _ = _tiny_gpu_and_oracle(lq, 2)
    y3, _, _ = _tiny_gpu_and_oracle(lq, 2)
    assert rel_err(y1, y2) <= 1e-6
    assert np.array_equal(y1.view(np.uint32), y1b.view(np.uint32))
    assert np.array_equal(y2.view(np.uint32), y3.view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 3, 33])
def test_linear_small_shapes(lq, bits, M):
    K, N = 512, 96
    say(f"linear A{bits} M={M}")
    rng = synth.seeded_rng(synth.TEST, 130, M, bits)
    P1 = synth.haar_orthogonal(16, rng)
    P2 = synth.haar_orthogonal(32, rng)
    x = synth.with_outliers(synth.gaussian((M, K), 131, M), 3, 15.0, 132, M)
    w = synth.gaussian((N, K), 133, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, bits)
    lq.loopq_w4a4_linear(dev(x), dev(P1), dev(P2), 0.9, bits, codes, scales, 32, N, y, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(w, 32)
    xt = gpu_xt(lq, dev(x), x, P1, P2)
    ref, _, _ = oracle.linear(xt, None, None, 0.9, bits, qw, sw, 32)
    assert rel_err(y.cpu().numpy(), ref) <= Y_TOL


def test_empty_input_is_a_no_op(lq):
    K, N = 256, 64
    w = synth.gaussian((N, K), 134, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.full((1, 0, N), 7.0, device="cuda")
    x = torch.empty((1, 0, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    lq.loopq_looped_forward(x, None, None, [1.0], 4, codes, scales, 32, N, y, 0, ws)
    torch.cuda.synchronize()


def test_zero_input_gives_zero_output(lq):
    K, N, M = 256, 64, 4
    w = synth.gaussian((N, K), 135, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.full((M, N), 7.0, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, 4)
    lq.loopq_w4a4_linear(torch.zeros((M, K), device="cuda"), None, None, 1.0, 4, codes, scales, 32,
                         N, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# ------------------------------------------------------------------------ fold

@pytest.mark.parametrize("n1,n2,N", [(16, 16, 128), (32, 64, 48), (64, 88, 6), (64, 108, 4)])
def test_fold_matches_oracle(lq, n1, n2, N):
    K = n1 * n2
    say(f"fold n1={n1} n2={n2} N={N}")
    rng = synth.seeded_rng(synth.TEST, 140, n1, n2)
    P1 = synth.haar_orthogonal(n1, rng)
    P2 = synth.haar_orthogonal(n2, rng)
    W = synth.gaussian((N, K), 141, N, scale=0.02)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_FOLD, 0, n1, K, n2, 0)
    lq.loopq_fold_weights(dev(W), dev(P1), dev(P2), out, ws)
    ref = oracle.fold_weights(W, P1, P2).astype(np.float32)
    got = out.cpu().numpy()
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert np.count_nonzero(ulps) <= max(2, K * N // 10000)


def test_fold_rejects_singular_factor(lq):
    P1 = np.eye(4, dtype=np.float32)
    P1[3] = P1[2]
    P2 = np.eye(8, dtype=np.float32)
    W = synth.gaussian((4, 32), 142, scale=0.02)
    out = torch.empty((4, 32), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_FOLD, 0, 4, 32, 8, 0)
    with pytest.raises(lq.LoopQError) as e:
        lq.loopq_fold_weights(dev(W), dev(P1), dev(P2), out, ws)
    assert e.value.status == lq.LOOPQ_ERR_SINGULAR


# ------------------------------------------------------------------------ decode (few rows)

@pytest.mark.parametrize("schedule", [1, 2])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("act,K,N", [("up_in", 2048, 96), ("down_in", 5632, 72)])
def test_decode_shapes(lq, act, K, N, M, bits, schedule):
    """Decode-sized calls (at most 16 rows per launch take the small-row
    kernel) at the block's factor shapes, against the oracle loop."""
    say(f"decode {act} K={K} N={N} M={M} A{bits} schedule={schedule}")
    wl = synth.ouro_block_workload(bits_a=bits, M=M, T=4)
    P1, P2 = synth.factors_for(wl, act, K)
    clips = synth.clips_for(wl, act)
    bits16, x32 = synth.activations_for(wl, act, K)
    w = synth.gaussian((N, K), 150, K, N, scale=0.02)
    codes, scales = pack(lq, w, 32)
    y = torch.empty((wl.T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, wl.T, M, K, N, bits)
    lq.loopq_looped_forward(bf16_dev(bits16), dev(P1), dev(P2), clips, bits, codes, scales, 32, N, y,
                            schedule, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(w, 32)
    T = wl.T
    xt = gpu_xt(lq, bf16_dev(bits16).view(T * M, K), x32.reshape(T * M, K), P1, P2).reshape(T, M, K)
    ref = oracle.looped_forward(xt, None, None, clips, bits, qw, sw, 32)
    assert rel_err(y.cpu().numpy(), ref) <= Y_TOL


def test_decode_graph_replays_match_eager(lq):
    """The few-row kernel keeps no state between launches (no work-group waits
    for another), so calls can be captured into a graph: every replay (with
    eager work between replays) equals the eager result bit for bit, and the
    eager result equals the oracle on the kernel's x~."""
    K, N, M, T = 2048, 200, 1, 4
    wl = synth.ouro_block_workload(bits_a=4, M=M, T=T)
    P1, P2 = synth.factors_for(wl, "up_in", K)
    clips = synth.clips_for(wl, "up_in")
    bits16, x32 = synth.activations_for(wl, "up_in", K)
    w = synth.gaussian((N, K), 160, K, N, scale=0.02)
    codes, scales = pack(lq, w, 32)
    x = bf16_dev(bits16)
    tP1, tP2 = dev(P1), dev(P2)
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4)
    y = torch.zeros((T, M, N), dtype=torch.float32, device="cuda")

    def step():
        for schedule in (1, 2):
            lq.loopq_looped_forward(x, tP1, tP2, clips, 4, codes, scales, 32, N, y, schedule, ws)

    step()
    torch.cuda.synchronize()
    eager = y.clone()
    qw, sw = oracle.quant_weights(w, 32)
    xt = gpu_xt(lq, x.view(T * M, K), x32.reshape(T * M, K), P1, P2).reshape(T, M, K)
    ref = oracle.looped_forward(xt, None, None, clips, 4, qw, sw, 32)
    assert rel_err(eager.cpu().numpy(), ref) <= Y_TOL
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep}"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, eager)


# ------------------------------------------------------------------------ loop-dependent sets

@pytest.mark.parametrize("M", [4, 16, 100])
def test_looped_forward_ex_matches_oracle(lq, M):
    """SLT-style loop-dependent weights and transforms and a per-loop activation
    bit width: loops [0, 1, 1, 0] use two sets (Haar factors; Hadamard factors,
    which make the transform the Walsh-Hadamard transform of order 2048) and
    widths [4, 8, 8, 4], against the oracle on each loop's kernel x~."""
    K, N, T = 2048, 160, 4
    say(f"looped_forward_ex M={M}")
    rng = synth.seeded_rng(synth.TEST, 180, M)
    F = [(synth.haar_orthogonal(32, rng), synth.haar_orthogonal(64, rng)),
         (synth.hadamard(32), synth.hadamard(64))]
    W = [synth.gaussian((N, K), 181, s, scale=0.02) for s in range(2)]
    packed = [pack(lq, w, 32) for w in W]
    qws = [oracle.quant_weights(w, 32) for w in W]
    sets, bits = [0, 1, 1, 0], [4, 8, 8, 4]
    clips = [0.9, 0.8, 0.7, 0.95]
    x = synth.with_outliers(synth.gaussian((T, M, K), 182, M), 8, 20.0, 183, M)
    bits16, x32 = synth.round_to_bf16(x)
    xd = bf16_dev(bits16)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_EX, T, M, K, N, 0)
    fd = [(dev(a), dev(b)) for a, b in F]
    lq.loopq_looped_forward_ex(xd, fd, clips, bits, packed, 32, N, y, sets, ws)
    torch.cuda.synchronize()
    # the oracle on each loop's x~ (the kernel's own, per set)
    xt = np.stack([gpu_xt(lq, xd[t], x32[t], *F[sets[t]]) for t in range(T)])
    ref = oracle.looped_forward_sets(xt, [(None, None)] * 2, clips, bits, qws, 32, sets)
    got = y.cpu().numpy()
    for t in range(T):
        assert rel_err(got[t], ref[t]) <= Y_TOL, t


@pytest.mark.parametrize("bits_a", [4, 8])
@pytest.mark.parametrize("M,sets,K,N,factors", [(64, [0, 1, 2, 3], 2048, 160, (32, 64)),
                                                (128, [0, 1, 1, 0], 2048, 160, (32, 64)),
                                                (64, [2, 0, 0, 1, 2, 1], 2048, 160, (32, 64)),
                                                (64, [1, 0, 1], 96, 40, (8, 12))])
def test_looped_forward_ex_grouped_gemm(lq, M, sets, K, N, factors, bits_a):
    """Loop-dependent weight sets at one bit width with M % 64 == 0 run as one
    grouped GEMM over all T * M rows (each loop's rows take its set's weights;
    each set's transform quantizes its loops' rows): against the oracle on
    each loop's kernel x~, and bitwise equal to running the loops one call
    each (the same kernels per tile)."""
    T = len(sets)
    say(f"grouped looped_forward_ex M={M} sets={sets} K={K} N={N} A{bits_a}")
    rng = synth.seeded_rng(synth.TEST, 185, M, T, K)
    nsets = max(sets) + 1
    F = [(synth.haar_orthogonal(factors[0], rng), synth.haar_orthogonal(factors[1], rng)) for _ in range(nsets)]
    W = [synth.gaussian((N, K), 186, si, K, scale=0.02) for si in range(nsets)]
    packed = [pack(lq, w, 32) for w in W]
    qws = [oracle.quant_weights(w, 32) for w in W]
    bits = [bits_a] * T
    clips = [0.95 - 0.05 * t for t in range(T)]
    x = synth.with_outliers(synth.gaussian((T, M, K), 187, M, T, K), min(8, K // 8), 20.0, 188, M)
    bits16, x32 = synth.round_to_bf16(x)
    xd = bf16_dev(bits16)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_EX, T, M, K, N, 0)
    fd = [(dev(a), dev(b)) for a, b in F]
    lq.loopq_looped_forward_ex(xd, fd, clips, bits, packed, 32, N, y, sets, ws)
    torch.cuda.synchronize()
    xt = np.stack([gpu_xt(lq, xd[t], x32[t], *F[sets[t]]) for t in range(T)])
    ref = oracle.looped_forward_sets(xt, [(None, None)] * nsets, clips, bits, qws, 32, sets)
    got = y.cpu().numpy()
    for t in range(T):
        assert rel_err(got[t], ref[t]) <= Y_TOL, t
    # loop by loop (one set per call: the ungrouped path) gives the same bits
    for t in range(T):
        y1 = torch.empty((1, M, N), dtype=torch.float32, device="cuda")
        ws1 = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_EX, 1, M, K, N, 0)
        lq.loopq_looped_forward_ex(xd[t:t + 1], [fd[sets[t]]], [clips[t]], [bits_a], [packed[sets[t]]], 32, N,
                                   y1, [0], ws1)
        torch.cuda.synchronize()
        assert torch.equal(y1[0], y[t]), t


def test_looped_forward_ex_with_one_set_is_the_shared_loop(lq):
    K, N, M, T = 512, 96, 40, 4
    P1, P2 = synth.hadamard(16), synth.hadamard(32)
    w = synth.gaussian((N, K), 184, scale=0.02)
    codes, scales = pack(lq, w, 32)
    x = dev(synth.gaussian((T, M, K), 185))
    clips = [0.9, 0.8, 0.7, 0.6]
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_EX, T, M, K, N, 0)
    y1 = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    lq.loopq_looped_forward_ex(x, [(dev(P1), dev(P2))], clips, [4] * T, [(codes, scales)], 32, N, y1,
                               [0] * T, ws)
    lq.loopq_looped_forward(x, dev(P1), dev(P2), clips, 4, codes, scales, 32, N, y2,
                            lq.LOOPQ_SCHED_WEIGHT_STATIONARY, ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
