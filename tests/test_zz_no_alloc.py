"""loopq_w4a4_linear_noalloc (the linear on the library's fixed scratch, for
callers that cannot allocate) against loopq_w4a4_linear on the same inputs:
the same kernels and layout, so the outputs must be bitwise equal.  Two
calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), then a third on yet another shape."""

import numpy as np
import pytest
import torch

from bit_ptq_looped_amd import synth

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(lq, M, K, N, factors, bits, dtype, key):
    rng = synth.seeded_rng(synth.TEST, 400, key)
    P1 = P2 = None
    if factors is not None:
        P1 = dev(synth.haar_orthogonal(factors[0], rng))
        P2 = dev(synth.haar_orthogonal(factors[1], rng))
    x = synth.with_outliers(synth.gaussian((M, K), 401, key), max(1, K // 100), 20.0, 402, key)
    if dtype == "bf16":
        bits16, _ = synth.round_to_bf16(x)
        xd = torch.from_numpy(bits16.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        xd = dev(x)
    w = synth.gaussian((N, K), 403, key, scale=0.02)
    codes, scales = lq.empty_packed_weights(K, N, 32)
    lq.loopq_pack_weights(dev(w), 32, codes, scales)
    return xd, P1, P2, codes, scales


def run_both(lq, M, K, N, factors, bits, dtype, key, clip=0.83):
    print(f"no-alloc linear M={M} K={K} N={N} factors={factors} A{bits} {dtype}", flush=True)
    xd, P1, P2, codes, scales = case(lq, M, K, N, factors, bits, dtype, key)
    y_ref = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LINEAR, 1, M, K, N, bits)
    lq.loopq_w4a4_linear(xd, P1, P2, clip, bits, codes, scales, 32, N, y_ref, ws)
    y = torch.full((M, N), -5.0, dtype=torch.float32, device="cuda")
    lq.loopq_w4a4_linear_noalloc(xd, P1, P2, clip, bits, codes, scales, 32, N, y)
    torch.cuda.synchronize()
    a, b = y.cpu().numpy(), y_ref.cpu().numpy()
    assert np.all(np.isfinite(a))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), float(np.max(np.abs(a - b)))


def test_noalloc_matches_the_linear_on_two_calls_then_a_third(lq):
    # first call: the GEMM path (300 rows, transform, W4A4) fills much of the scratch
    run_both(lq, 300, 2048, 512, (32, 64), 4, "bf16", 1)
    # second, smaller: the few-row path (5 rows, A8), on the scratch the first call left
    run_both(lq, 5, 256, 96, (16, 16), 8, "f32", 2)
    # third: GEMM path again, no transform, ragged rows
    run_both(lq, 77, 160, 40, None, 4, "f32", 3)


def test_noalloc_rejects_a_call_larger_than_the_scratch(lq):
    K = N = 2048
    M = 32768  # needs more than the 64 MiB scratch
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    codes, scales = lq.empty_packed_weights(K, N, 32)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(lq.LoopQError) as e:
        lq.loopq_w4a4_linear_noalloc(x, None, None, 1.0, 4, codes, scales, 32, N, y)
    assert e.value.status == lq.LOOPQ_ERR_WORKSPACE
