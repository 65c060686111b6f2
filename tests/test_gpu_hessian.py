"""GPU parity of the trajectory Hessian accumulation (``loopq_hessian_accumulate``)
against the CPU oracle, through the C ABI.

Bar, derived from the arithmetic (``xt_check.hessian_bound``): the kernel takes
each product x~_ri x~_rj as the six bf16-plane products of order <= 2 (each
exact in fp32, the dropped rest below 2^-20 of |x~_ri x~_rj|) and adds them in
fp32 (six additions per row, one per split-tile piece, one into H), so every
element of H0 + X^T X lies within
gamma(6 rows + ceil(rows / 64) + 2) ((1 + 2^-6) |X|^T |X| + |H0|) + 2^-20 |X|^T |X|
of the exact value, which the fp64 oracle gives (its own error is far below
that).  Several calls chain: the bound adds up over them.  H is exactly
symmetric (one value stored at (i, j) and (j, i)) and the call is
deterministic.
"""

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from xt_check import check_xt, hessian_bound

pytestmark = pytest.mark.gpu

def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(*a):
    print(*a, flush=True)


def workspace(lq, rows, K):
    n = lq.loopq_workspace_bytes(lq.LOOPQ_OP_HESSIAN, 0, rows, K, 0, 0)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")


def accumulate(lq, xs, H0):
    """H0 + sum over the row blocks xs (one call each) on the GPU, fp32."""
    K = H0.shape[0]
    H = dev(H0.astype(np.float32))
    ws = workspace(lq, max(x.shape[0] for x in xs), K)
    for x in xs:
        lq.loopq_hessian_accumulate(dev(x.astype(np.float32)), H, ws)
    torch.cuda.synchronize()
    return H.cpu().numpy()


def check_bound(got, xs, H0):
    """Element-wise bound of the module docstring over a chain of calls: each
    call's bound with the running |H| before it as its |H0|."""
    want = np.asarray(H0, dtype=np.float64) + sum(oracle.trajectory_hessian(x) for x in xs)
    run = np.abs(np.asarray(H0, dtype=np.float64))
    bound = np.zeros_like(run)
    for x in xs:
        mag_x = oracle.trajectory_hessian(np.abs(x))
        bound = bound + hessian_bound(x.shape[0], mag_x, run)
        run = run + mag_x
    err = np.abs(got.astype(np.float64) - want)
    ratio = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), f"H outside the plane-product accumulation bound (max error/bound {ratio:.3g})"
    return ratio


def random_symmetric(K, *key):
    a = synth.gaussian((K, K), *key)
    return ((a + a.T) * np.float32(0.5)).astype(np.float32)


# (rows, K), tiles of 128: one tile and one row; a ragged column edge (K % 128
# of 96, 64, 32) and ragged rows; fewer tiles than work groups with each tile
# split across many of them (K = 256: 3 tiles; K = 2048: 136); whole tiles plus
# split leftovers (K = 4160: 561 tiles, K = 5632: 990).
@pytest.mark.parametrize("rows,K", [(1, 32), (63, 96), (130, 256), (4096, 256), (333, 2048),
                                    (1000, 4160), (77, 4128), (70, 5632)])
def test_hessian_matches_oracle(lq, rows, K):
    say(f"hessian rows={rows} K={K}")
    x = synth.with_outliers(synth.gaussian((rows, K), 71, rows, K), max(1, K // 100), 20.0, 72, K)
    H0 = random_symmetric(K, 73, K) if rows > 1 else np.zeros((K, K), np.float32)
    got = accumulate(lq, [x], H0)
    ratio = check_bound(got, [x], H0)
    say(f"  max error / bound {ratio:.3g}")
    assert np.array_equal(got, got.T)
    again = accumulate(lq, [x], H0)
    assert np.array_equal(got, again)


def test_hessian_without_rows_is_a_no_op(lq):
    K = 256
    H0 = random_symmetric(K, 74)
    H = dev(H0)
    lq.loopq_hessian_accumulate(torch.empty((0, K), dtype=torch.float32, device="cuda"), H, workspace(lq, 0, K))
    torch.cuda.synchronize()
    assert np.array_equal(H.cpu().numpy(), H0)


def test_hessian_of_loop_trajectory_from_quantizer_dumps(lq):
    """The side output of a looped forward: the x~ rows every loop quantizes
    (the quantizer's dump), accumulated one loop per call, against the oracle's
    trajectory Hessian of those rows (Ouro-like qkv input, K = 2048 = 32 x 64)."""
    wl = synth.ouro_block_workload(M=96)
    K = 2048
    P1, P2 = synth.factors_for(wl, "qkv_in", K)
    bits, x32 = synth.activations_for(wl, "qkv_in", K)
    T, M = x32.shape[0], x32.shape[1]
    p1, p2 = dev(P1), dev(P2)
    H = torch.zeros((K, K), dtype=torch.float32, device="cuda")
    ws = workspace(lq, M, K)
    dumps = []
    for t in range(T):
        say(f"loop {t}")
        xt = torch.from_numpy(np.ascontiguousarray(bits[t]).view(np.int16)).cuda().view(torch.bfloat16)
        codes = torch.empty((M, K), dtype=torch.int8, device="cuda")
        steps = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
        dump = torch.empty((M, K), dtype=torch.float32, device="cuda")
        lq.loopq_quant_act(xt, p1, p2, 1.0, 4, codes, steps, dump)
        lq.loopq_hessian_accumulate(dump, H, ws)
        torch.cuda.synchronize()
        d = dump.cpu().numpy()
        check_xt(d, x32[t], P1, P2)
        dumps.append(d)
    got = H.cpu().numpy()
    ratio = check_bound(got, dumps, np.zeros((K, K)))
    say(f"  max error / bound {ratio:.3g}")
    assert np.array_equal(got, got.T)


def test_hessian_rank_grows_along_a_drifting_trajectory(lq):
    """Thresholded rank (1e-3 lambda_max, "Quantizing Looped Transformers",
    Table 1) of the accumulated Hessian after each loop: loop t's rows span
    43 + 8 t fixed directions, so the rank after loop t is 43 + 8 t for the
    GPU's fp32 H and for the oracle's fp64 H alike.  Orthonormal directions
    and 512 rows per loop keep the smallest nonzero eigenvalue above 1/20 of
    the largest, far from the threshold."""
    K, M, T, d0, dd = 512, 512, 4, 43, 8
    basis = synth.haar_orthogonal(K, synth.seeded_rng(synth.TEST, 75))[: d0 + dd * (T - 1)]
    H = torch.zeros((K, K), dtype=torch.float32, device="cuda")
    ws = workspace(lq, M, K)
    xs = []
    for t in range(T):
        d = d0 + dd * t
        z = synth.gaussian((M, d), 76, t)
        x = (z.astype(np.float64) @ basis[:d].astype(np.float64)).astype(np.float32)
        xs.append(x)
        lq.loopq_hessian_accumulate(dev(x), H, ws)
        torch.cuda.synchronize()
        got = H.cpu().numpy()
        want_rank = oracle.thresholded_rank(oracle.trajectory_hessian(xs))
        assert want_rank == d
        assert oracle.thresholded_rank(got) == d


@pytest.mark.parametrize("schedule,M", [(2, 96), (1, 96), (2, 3), (1, 3)])
def test_looped_forward_hessian_side_output(lq, schedule, M):
    """loopq_looped_forward_hessian: the forward's own quantizer writes the x~
    it quantizes (bitwise loopq_quant_act's dump of the same rows) and H0 +
    x~^T x~ over all loops is bitwise one loopq_hessian_accumulate call on
    those rows; y is bitwise the plain looped forward's where that call also
    takes the quantizer and the GEMM, and matches the oracle on x~ (1e-4)."""
    wl = synth.ouro_block_workload(M=M)
    K, N = 2048, 256
    P1, P2 = synth.factors_for(wl, "qkv_in", K)
    bits, x32 = synth.activations_for(wl, "qkv_in", K)
    T = x32.shape[0]
    clips = [1.0, 0.9, 0.95, 0.85][:T]
    say(f"forward + hessian schedule={schedule} T={T} M={M}")
    W = synth.gaussian((N, K), 950, M, scale=0.02)
    wt = oracle.fold_weights(W, P1, P2).astype(np.float32)
    qw, sw = oracle.quant_weights(wt, 32)
    codes, scales = lq.empty_packed_weights(K, N, 32)
    lq.loopq_pack_weights(dev(wt), 32, codes, scales)
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    p1, p2 = dev(P1), dev(P2)
    H0 = random_symmetric(K, 951)
    H = dev(H0.astype(np.float32))
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_HESSIAN, T, M, K, N, 4)
    lq.loopq_looped_forward_hessian(x, p1, p2, clips, 4, codes, scales, 32, N, y, schedule, H, ws)
    torch.cuda.synchronize()
    base = lq.loopq_workspace_bytes(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4)
    off = (base + 255) // 256 * 256
    xt_ws = ws[off:off + T * M * K * 4].view(torch.float32).view(T * M, K).clone()
    # the same rows through loopq_quant_act (one call per loop: its own clip)
    dump = torch.empty((T * M, K), dtype=torch.float32, device="cuda")
    for t in range(T):
        codes_t = torch.empty((M, K), dtype=torch.int8, device="cuda")
        steps_t = torch.empty((M, K // 32), dtype=torch.float32, device="cuda")
        lq.loopq_quant_act(x[t], p1, p2, clips[t], 4, codes_t, steps_t, dump[t * M:(t + 1) * M])
    H2 = dev(H0.astype(np.float32))
    lq.loopq_hessian_accumulate(dump, H2, workspace(lq, T * M, K))
    y2 = torch.empty_like(y)
    lq.loopq_looped_forward(x, p1, p2, clips, 4, codes, scales, 32, N, y2, schedule,
                            lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4))
    torch.cuda.synchronize()
    assert torch.equal(xt_ws, dump)
    assert torch.equal(H, H2)
    d = dump.cpu().numpy()
    check_xt(d, x32.reshape(T * M, K), P1, P2)
    ratio = check_bound(H.cpu().numpy(), [d], H0)
    say(f"  H max error / bound {ratio:.3g}")
    rows_per_launch = T * M if schedule == 2 else M
    if rows_per_launch > 16:
        assert torch.equal(y, y2)
    ref = oracle.looped_forward(d.reshape(T, M, K), None, None, clips, 4, qw, sw, 32)
    got = y.cpu().numpy().astype(np.float64)
    assert float(np.max(np.abs(got - ref)) / np.max(np.abs(ref))) <= 1e-4
