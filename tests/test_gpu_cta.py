"""GPU parity of the CTA loop-transition adapter ("paper_specification.yaml",
``loopq_components.cta``, Section 4.3, Eq.(7); ``cta_rank: 8``; reading S20:
h -> a * h + b + eta * U (V^T h) at the transition into loop t >= 1).

The kernel's adapted rows are compared with the oracle's fp64 map: within an
fp32 accumulation bound of it (fp32 state), plus half a bf16 ulp for a bf16
state.  Cases the fp32 arithmetic decides exactly are bitwise: identity
parameters return the input, a zero gate returns fl32(a h + b) (rounded to
bf16 for a bf16 state), in place equals out of place.  The looped forward
with CTA is checked like the plain one (S15): y against the oracle applied
to the kernel's x~ of the kernel's adapted rows, and with identity
parameters it is bitwise the plain looped forward."""

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth
from test_gpu_parity import Y_TOL, dev, rel_err, say
from xt_check import gpu_xt

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def cta_params(K, r, ntr, key):
    rng = synth.seeded_rng(synth.TEST, 900, K, r, ntr, key)
    U = (rng.standard_normal((K, r)) / np.sqrt(K)).astype(np.float32)
    V = (rng.standard_normal((K, r)) / np.sqrt(K)).astype(np.float32)
    a = (1.0 + 0.1 * rng.standard_normal((ntr, K))).astype(np.float32)
    b = (0.05 * rng.standard_normal((ntr, K))).astype(np.float32)
    eta = [float(v) for v in np.float32(rng.uniform(-1.0, 1.0, ntr))]
    return U, V, a, b, eta


def state_values(shape, key, state):
    x = synth.gaussian(shape, 910, key)
    return oracle.round_bf16(x).astype(np.float32) if state == "bf16" else x.astype(np.float32)


def to_dev(x32, state):
    t = dev(x32)
    return t.to(torch.bfloat16) if state == "bf16" else t


def cta_bound(h, U, V, a, b, eta, state):
    """The oracle's map and the bound the kernel's result must keep to it."""
    h = np.asarray(h, dtype=np.float64)
    K, r = U.shape
    exact = oracle.cta_transition(h, U, V, a, b, eta)
    z = h @ V.astype(np.float64)
    s = z @ U.astype(np.float64).T
    aU, aV = np.abs(U.astype(np.float64)), np.abs(V.astype(np.float64))
    dz = (K + 16) * U32 * (np.abs(h) @ aV)                     # V^T h in fp32, fixed order
    es = dz @ aU.T + (r + 1) * U32 * (np.abs(z) @ aU.T)          # sum_j U z_j
    e32 = 3 * U32 * (np.abs(a * h) + np.abs(b) + abs(eta) * np.abs(s)) + abs(eta) * es
    if state == "bf16":
        mag = np.maximum(np.abs(exact) + e32, 2.0 ** -126)
        return exact, e32 + 0.5 * np.exp2(np.floor(np.log2(mag)) - 7)
    return exact, e32


def cta_gpu(lq, hdev, U, V, a, b, eta, out=None):
    out = torch.empty_like(hdev) if out is None else out
    lq.loopq_cta_apply(hdev, dev(U), dev(V), dev(a), dev(b), eta, out)
    torch.cuda.synchronize()
    return out


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("state,M,K,r", [("bf16", 37, 2560, 8), ("fp32", 7, 256, 3), ("bf16", 1, 6912, 16),
                                         ("fp32", 37, 6912, 8), ("bf16", 7, 256, 1), ("fp32", 5, 17920, 8),
                                         ("bf16", 45, 3072, 8), ("fp32", 19, 2080, 8), ("bf16", 16, 2080, 5),
                                         ("fp32", 9, 3072, 8), ("bf16", 33, 3104, 8), ("bf16", 21, 2080, 8)])
def test_cta_apply_within_bound_of_the_oracle(lq, state, M, K, r):
    say(f"cta apply {state} M={M} K={K} r={r}")
    U, V, a, b, eta = cta_params(K, r, 1, M)
    h = state_values((M, K), K + r, state)
    got = host(cta_gpu(lq, to_dev(h, state), U, V, a[0], b[0], eta[0]))
    exact, bound = cta_bound(h, U, V, a[0], b[0], eta[0], state)
    err = np.abs(got - exact)
    assert np.all(err <= bound), f"max err/bound {float(np.max(err / bound)):.3f}"
    # the bound is tight enough to see a dropped low-rank term
    assert np.max(np.abs(exact - oracle.cta_transition(h, U, V, a[0], b[0], 0.0)) / bound) > 10


@pytest.mark.parametrize("K", [512, 2080, 3584])
@pytest.mark.parametrize("state", ["bf16", "fp32"])
def test_cta_identity_zero_gate_and_in_place(lq, state, K):
    M, r = 9, 8
    U, V, a, b, eta = cta_params(K, r, 1, 77)
    h = state_values((M, K), 78, state)
    hd = to_dev(h, state)
    # identity: the rows come back bitwise
    got = cta_gpu(lq, hd, U, V, np.ones((1, K), np.float32)[0], np.zeros(K, np.float32), 0.0)
    assert torch.equal(got, hd)
    # zero gate: one fp32 rounding of a h + b (exact in fp64), then the state's
    got = host(cta_gpu(lq, hd, U, V, a[0], b[0], 0.0))
    want = (a[0].astype(np.float64) * h + b[0]).astype(np.float32).astype(np.float64)
    if state == "bf16":
        want = oracle.round_bf16(want)
    np.testing.assert_array_equal(got, want)
    # in place equals out of place, bitwise
    ref = cta_gpu(lq, hd, U, V, a[0], b[0], eta[0])
    inplace = hd.clone()
    cta_gpu(lq, inplace, U, V, a[0], b[0], eta[0], out=inplace)
    assert torch.equal(inplace, ref)


def _forward_case(lq, T, M, K, N, n1, n2, state, key):
    rng = synth.seeded_rng(synth.TEST, 920, T, M, K, N, key)
    P1, P2 = synth.haar_orthogonal(n1, rng), synth.haar_orthogonal(n2, rng)
    W = synth.gaussian((N, K), 921, key, scale=0.02)
    wt = oracle.fold_weights(W, P1, P2).astype(np.float32)
    qw, sw = oracle.quant_weights(wt, 32)
    codes, scales = lq.empty_packed_weights(K, N, 32)
    lq.loopq_pack_weights(dev(wt), 32, codes, scales)
    xs = state_values((T, M, K), key, state)
    clips = [1.0, 0.9, 0.95, 0.85, 1.0, 0.8, 0.9, 0.97][:T]
    return P1, P2, qw, sw, codes, scales, xs, clips


@pytest.mark.parametrize("state,T,M,schedule", [("bf16", 4, 64, 2), ("bf16", 4, 64, 1), ("fp32", 3, 16, 1),
                                                ("bf16", 4, 1, 1), ("fp32", 2, 40, 2)])
def test_looped_forward_cta_matches_oracle(lq, state, T, M, schedule):
    K, N, n1, n2 = 2048, 256, 32, 64
    say(f"looped forward cta {state} T={T} M={M} schedule={schedule}")
    P1, P2, qw, sw, codes, scales, xs, clips = _forward_case(lq, T, M, K, N, n1, n2, state, 1 + M)
    U, V, a, b, eta = cta_params(K, 8, T - 1, T * M)
    xd = to_dev(xs, state)
    y = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_CTA, T, M, K, N, 4)
    lq.loopq_looped_forward_cta(xd, dev(P1), dev(P2), clips, 4, codes, scales, 32, N, y, schedule,
                                dev(U), dev(V), dev(a), dev(b), eta, ws)
    torch.cuda.synchronize()
    # the kernel's adapted loop inputs, each within the bound of the oracle's map
    adapted = [xd[0]]
    for t in range(1, T):
        out = cta_gpu(lq, xd[t], U, V, a[t - 1], b[t - 1], eta[t - 1])
        exact, bound = cta_bound(xs[t], U, V, a[t - 1], b[t - 1], eta[t - 1], state)
        assert np.all(np.abs(host(out) - exact) <= bound), f"loop {t}"
        adapted.append(out)
    ad = torch.stack(adapted)
    ad32 = host(ad).astype(np.float32)
    xt = gpu_xt(lq, ad.view(T * M, K), ad32.reshape(T * M, K), P1, P2).reshape(T, M, K)
    ref = oracle.looped_forward(xt, None, None, clips, 4, qw, sw, 32)
    got = y.cpu().numpy()
    assert rel_err(got, ref) <= Y_TOL
    for t in range(T):
        assert rel_err(got[t], ref[t]) <= Y_TOL
    # the adapter changed loops 1.. (not a no-op), and loop 0 is the plain loop
    plain = oracle.looped_forward(gpu_xt(lq, xd.reshape(T * M, K), xs.reshape(T * M, K), P1, P2).reshape(T, M, K),
                                  None, None, clips, 4, qw, sw, 32)
    assert rel_err(got[0], plain[0]) <= Y_TOL
    assert rel_err(got[T - 1], plain[T - 1]) > 1e-2


@pytest.mark.parametrize("schedule", [1, 2])
@pytest.mark.parametrize("M", [16, 64])
def test_identity_cta_is_bitwise_the_plain_looped_forward(lq, schedule, M):
    T, K, N = 4, 2048, 256
    say(f"identity cta T={T} M={M} schedule={schedule}")
    P1, P2, qw, sw, codes, scales, xs, clips = _forward_case(lq, T, M, K, N, 32, 64, "bf16", 5)
    U, V, _, _, _ = cta_params(K, 8, T - 1, 5)
    a, b, eta = np.ones((T - 1, K), np.float32), np.zeros((T - 1, K), np.float32), [0.0] * (T - 1)
    xd = to_dev(xs, "bf16")
    y1 = torch.empty((T, M, N), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    ws = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD_CTA, T, M, K, N, 4)
    lq.loopq_looped_forward_cta(xd, dev(P1), dev(P2), clips, 4, codes, scales, 32, N, y1, schedule,
                                dev(U), dev(V), dev(a), dev(b), eta, ws)
    ws2 = lq.empty_workspace(lq.LOOPQ_OP_LOOPED_FORWARD, T, M, K, N, 4)
    lq.loopq_looped_forward(xd, dev(P1), dev(P2), clips, 4, codes, scales, 32, N, y2, schedule, ws2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # one loop: no transition at all
    y3 = torch.empty((1, M, N), dtype=torch.float32, device="cuda")
    y4 = torch.empty_like(y3)
    U2, V2, a2, b2, e2 = cta_params(K, 8, 1, 6)
    lq.loopq_looped_forward_cta(xd[:1], dev(P1), dev(P2), clips[:1], 4, codes, scales, 32, N, y3, schedule,
                                dev(U2), dev(V2), dev(a2), dev(b2), e2, ws)
    lq.loopq_looped_forward(xd[:1], dev(P1), dev(P2), clips[:1], 4, codes, scales, 32, N, y4, schedule, ws2)
    torch.cuda.synchronize()
    assert torch.equal(y3, y4)
