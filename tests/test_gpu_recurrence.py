"""GPU parity of the dependent adapter recurrence (``loopq_recurrent_adapter``)
against the CPU oracle, through the C ABI.

A recurrence amplifies the fp32 rounding differences of one loop through the
quantizer's decisions in the next, so each loop is checked on its own input:
loop t's output y[t] against the oracle's linear on cat(s_t, e), with s_t the
state the GPU produced (s_0 for t = 0, else y[t - 1]); bar as for one linear,
max|y - y_oracle| / max|y_oracle| <= 1e-4.  With a transform the oracle
quantizes the kernel's x~ of those rows (fp32-class bound checked first).
"""

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from xt_check import gpu_xt

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


# (M, N, gw, bits, factors): one row (quantized in place by the few-row
# kernel), 16 rows, the GEMM path; N % 32 == 16 puts a 32-group across the
# s / e boundary; g_w = 128 with a short last weight group; a transform over
# K = 2N
@pytest.mark.parametrize("M,N,gw,bits,factors", [(1, 64, 32, 4, None), (16, 80, 32, 8, None),
                                                 (100, 160, 128, 8, None), (4, 64, 32, 4, (8, 16)),
                                                 (48, 1024, 32, 4, (32, 64))])
def test_recurrent_adapter_matches_oracle_loop_by_loop(lq, M, N, gw, bits, factors):
    T = 5
    say(f"recurrence M={M} N={N} gw={gw} A{bits} factors={factors}")
    K = 2 * N
    P1 = P2 = None
    if factors:
        rng = synth.seeded_rng(synth.TEST, 210, *factors)
        P1, P2 = synth.haar_orthogonal(factors[0], rng), synth.haar_orthogonal(factors[1], rng)
    s0 = synth.gaussian((M, N), 211, M, N)
    e = synth.with_outliers(synth.gaussian((M, N), 212, M, N), 2, 10.0, 213)
    # a contracting map keeps the state's scale steady over the loops
    w = synth.gaussian((N, K), 214, N, K, scale=0.5 / np.sqrt(K))
    clips = [1.0 - 0.05 * t for t in range(T)]
    codes, scales = pack(lq, w, gw)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, M, 0, N, bits),
                     dtype=torch.uint8, device="cuda")
    lq.loopq_recurrent_adapter(dev(s0), dev(e), None if P1 is None else dev(P1), None if P2 is None else dev(P2),
                               clips, bits, codes, scales, gw, y, ws)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    qw, sw = oracle.quant_weights(w, gw)
    for t in range(T):
        state = s0 if t == 0 else got[t - 1]
        x = np.concatenate([state, e], axis=1).astype(np.float32)
        xt = gpu_xt(lq, dev(x), x, P1, P2)
        ref, _, _ = oracle.linear(xt, None, None, clips[t], bits, qw, sw, gw)
        err = rel_err(got[t], ref)
        say(f"  loop {t}: rel err {err:.2e}, max|y| {np.max(np.abs(ref)):.3g}")
        assert err <= Y_TOL
    assert np.all(np.isfinite(got))


def test_recurrent_adapter_feeds_the_state_back(lq):
    """W = [7 I | 0] (e meets zero weights): the GPU recurrence equals the
    oracle's whole recurrence s_{t+1} = 7 * RTN(s_t) exactly, and loop t + 1
    differs from loop t (the state is fed back, not the first input)."""
    M, N, T = 2, 64, 3
    s0 = synth.gaussian((M, N), 215)
    e = synth.gaussian((M, N), 216, scale=5.0)
    W = np.zeros((N, 2 * N), dtype=np.float32)
    W[:, :N] = 7.0 * np.eye(N, dtype=np.float32)
    codes, scales = pack(lq, W, 32)
    clips = [1.0, 0.8, 0.9]
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(lq.loopq_workspace_bytes(lq.LOOPQ_OP_RECURRENT_ADAPTER, 0, M, 0, N, 4),
                     dtype=torch.uint8, device="cuda")
    lq.loopq_recurrent_adapter(dev(s0), dev(e), None, None, clips, 4, codes, scales, 32, y, ws)
    torch.cuda.synchronize()
    qw, sw = oracle.quant_weights(W, 32)
    want = oracle.recurrent_adapter(s0, e, None, None, clips, 4, qw, sw, 32)
    got = y.cpu().numpy()
    np.testing.assert_array_equal(got, want)
    assert not np.array_equal(got[1], got[0])


def test_recurrent_adapter_without_rows_is_a_no_op(lq):
    N = 64
    codes, scales = pack(lq, synth.gaussian((N, 2 * N), 217, scale=0.1), 32)
    y = torch.full((2, 1, N), 3.0, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    empty = torch.empty((0, N), dtype=torch.float32, device="cuda")
    lq.loopq_recurrent_adapter(empty, empty, None, None, [1.0, 1.0], 4, codes, scales, 32, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)
