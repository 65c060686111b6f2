"""GPU parity of the per-token activation steps (the rtn_w4a4_per_token arm of
"The arms") against the CPU oracle, through the C ABI.

Bars as for the group path: codes and steps bit-exact (the step repeated in
every group slot of its row), y within 1e-4 of max|y|; with a transform the
kernel's x~ dump is first checked against the fp32-class bound, and the oracle
quantizes that dump.
"""

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


def say(*a):
    print(*a, flush=True)


def rel_err(y, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(y, dtype=np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def pack(lq, w32, gw):
    N, K = w32.shape
    codes, scales = lq.empty_packed_weights(K, N, gw)
    lq.loopq_pack_weights(dev(w32), gw, codes, scales)
    return codes, scales


def quant_token_gpu(lq, xdev, P1, P2, clip, bits, with_xt):
    M, K = xdev.shape
    codes = torch.empty((M, K), dtype=torch.int8, device="cuda")
    scales = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((M, K), dtype=torch.float32, device="cuda") if with_xt else None
    lq.loopq_quant_act_per_token(xdev, None if P1 is None else dev(P1), None if P2 is None else dev(P2),
                                 clip, bits, codes, scales, xt)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), (xt.cpu().numpy() if with_xt else None)


def x_dev_and_f32(M, K, dtype, key):
    x = synth.with_outliers(synth.gaussian((M, K), 200, key, M, K), max(1, K // 100), 25.0, 201, key)
    if dtype == "bf16":
        bits, x32 = synth.round_to_bf16(x)
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16), x32
    return dev(x), x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M,K", [(1, 32), (7, 256), (33, 2048), (5, 5632)])
def test_quant_per_token_plain(lq, dtype, bits, M, K):
    say(f"per-token {dtype} A{bits} M={M} K={K}")
    xdev, x32 = x_dev_and_f32(M, K, dtype, 1)
    codes, scales, _ = quant_token_gpu(lq, xdev, None, None, 0.85, bits, False)
    qa, sa = oracle.quant_act(x32, 0.85, bits, group=K)
    np.testing.assert_array_equal(codes, qa.astype(np.int8))
    np.testing.assert_array_equal(scales, np.repeat(sa, K // 32, axis=1))


@pytest.mark.parametrize("n1,n2", [(32, 64), (64, 88)])
def test_quant_per_token_transformed(lq, n1, n2):
    K, M = n1 * n2, 12
    say(f"per-token transform ({n1},{n2})")
    rng = synth.seeded_rng(synth.TEST, 202, n1, n2)
    P1, P2 = synth.haar_orthogonal(n1, rng), synth.haar_orthogonal(n2, rng)
    xdev, x32 = x_dev_and_f32(M, K, "bf16", 2)
    codes, scales, xt = quant_token_gpu(lq, xdev, P1, P2, 0.7, 4, True)
    check_xt(xt, x32, P1, P2)
    qa, sa = oracle.quant_act(xt, 0.7, 4, group=K)
    np.testing.assert_array_equal(codes, qa.astype(np.int8))
    np.testing.assert_array_equal(scales, np.repeat(sa, K // 32, axis=1))
    # without the x~ output (x~ then stays on chip): the same codes and steps
    codes2, scales2, _ = quant_token_gpu(lq, xdev, P1, P2, 0.7, 4, False)
    np.testing.assert_array_equal(codes2, codes)
    np.testing.assert_array_equal(scales2, scales)


def test_quant_per_token_zero_row_and_saturation(lq):
    K = 256
    x = synth.gaussian((3, K), 203)
    x[1] = 0.0                      # step 0, codes 0
    x[2, 7] = 1e4                   # one huge element: every other code rounds to 0
    codes, scales, _ = quant_token_gpu(lq, dev(x), None, None, 0.5, 4, False)
    qa, sa = oracle.quant_act(x, 0.5, 4, group=K)
    np.testing.assert_array_equal(codes, qa.astype(np.int8))
    np.testing.assert_array_equal(scales, np.repeat(sa, K // 32, axis=1))
    assert np.all(scales[1] == 0) and np.all(codes[1] == 0)
    assert codes[2, 7] == 7             # clip 0.5 saturates the maximum at qmax


# (T, M, K, N, gw, factors): the few-row kernel (T*M <= 16) and the MFMA GEMM,
# both code formats (A4 fp6 operands, A8 INT8), weight groups of 32 and 128;
# every loop with its own clip
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T,M,K,N,gw,factors", [(1, 3, 512, 96, 32, (16, 32)), (4, 4, 2048, 200, 32, (32, 64)),
                                                (3, 100, 2048, 160, 32, (32, 64)), (1, 70, 640, 64, 128, None),
                                                (2, 40, 5632, 72, 32, (64, 88))])
def test_looped_per_token_matches_oracle(lq, bits, T, M, K, N, gw, factors):
    say(f"per-token loop A{bits} T={T} M={M} K={K} N={N} gw={gw} factors={factors}")
    P1 = P2 = None
    if factors:
        rng = synth.seeded_rng(synth.TEST, 204, *factors)
        P1, P2 = synth.haar_orthogonal(factors[0], rng), synth.haar_orthogonal(factors[1], rng)
    xdev, x32 = x_dev_and_f32(T * M, K, "bf16", 3)
    clips = [0.95 - 0.1 * t for t in range(T)]
    w = synth.gaussian((N, K), 205, N, K, scale=0.02)
    codes, scales = pack(lq, w, gw)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, T, M, K, N, bits)
    lq.loopq_looped_forward_per_token(xdev.view(T, M, K), None if P1 is None else dev(P1),
                                      None if P2 is None else dev(P2), clips, bits, codes, scales, gw, N, y, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(w, gw)
    xt = gpu_xt(lq, xdev, x32, P1, P2).reshape(T, M, K)
    got = y.cpu().numpy()
    for t in range(T):
        ref, _, _ = oracle.linear_per_token(xt[t], None, None, clips[t], bits, qw, sw, gw)
        err = rel_err(got[t], ref)
        say(f"  loop {t}: rel err {err:.2e}")
        assert err <= Y_TOL
        # per token differs from the group-32 arm on these outlier rows
        ref_g, _, _ = oracle.linear(xt[t], None, None, clips[t], bits, qw, sw, gw)
        assert rel_err(ref, ref_g) > 1e-3


def test_looped_per_token_empty_is_a_no_op(lq):
    K, N = 256, 64
    codes, scales = pack(lq, synth.gaussian((N, K), 206, scale=0.02), 32)
    y = torch.full((1, 1, N), 5.0, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN, 1, 1, K, N, 4)
    lq.loopq_looped_forward_per_token(torch.empty((1, 0, K), dtype=torch.float32, device="cuda"), None, None, [1.0],
                                      4, codes, scales, 32, N, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 5.0)
