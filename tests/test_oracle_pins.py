"""Pins of the CPU oracle against things other than itself.

Hand-derived Eq.(4) examples (tests/golden), brute force over small groups,
closed forms and invariants (orthogonality, the fold identity, Kronecker
products from numpy), exact rational arithmetic for the fp32/fp16 roundings,
and special cases that reduce to a plain library product.  Sources: the LoopQ
reproduction's paper_specification.yaml (lq1_quantization Eq.(4),
loopq_components, implementation_status lq2/lq3) and its README ("The arms").
"""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_ptq_looped_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "eq4_hand_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _pad32(vals):
    g = np.zeros((1, 32), dtype=np.float32)
    g[0, :len(vals)] = np.array(vals, dtype=np.float32)
    return g


# ---------------------------------------------------------------- Eq.(4) by hand

@pytest.mark.parametrize("case", _golden()["activation_groups"], ids=lambda c: c["id"])
def test_eq4_hand_examples(case):
    x = _pad32(case["x"])
    q, s = oracle.quant_act(x, case["clip"], case["bits"])
    assert s.shape == (1, 1)
    assert s[0, 0] == np.float32(case["step"])
    want = np.zeros(32, dtype=np.int64)
    want[:len(case["codes"])] = case["codes"]
    np.testing.assert_array_equal(q[0].astype(np.int64), want)


def test_weight_step_is_fp16_rounded_before_codes():
    case = _golden()["weight_groups"][0]
    w = _pad32(case["w"])
    q, s16 = oracle.quant_weights(w, 32)
    assert int(s16.view(np.uint16)[0, 0]) == case["step_fp16_bits"]
    np.testing.assert_array_equal(q[0, :6].astype(np.int64), case["codes"])
    # the same group quantized with the unrounded fp32 step differs (order matters)
    s32 = (np.max(np.abs(w)) / np.float32(7)).astype(np.float32)
    alt = np.clip(np.rint((w[0, :6] / s32).astype(np.float32)), -7, 7).astype(np.int64)
    np.testing.assert_array_equal(alt, case["codes_if_fp32_step"])


def test_hand_dot():
    case = _golden()["dot_examples"][0]
    a = np.array(case["a"], dtype=np.int8)[None, :]
    w = np.array(case["w"], dtype=np.int8)[None, :]
    d = oracle.group_dots(np.pad(a, ((0, 0), (0, 24))), np.pad(w, ((0, 0), (0, 24))))
    assert d.shape == (1, 1, 1) and int(d[0, 0, 0]) == case["dot"]


# ---------------------------------------------------------------- brute force

def _brute_codes(v, qmax):
    """argmin over the integer grid of |v - q|, ties to the even q (no rint)."""
    qs = np.arange(-qmax, qmax + 1, dtype=np.float64)
    dist = np.abs(v.astype(np.float64)[..., None] - qs)   # exact: v is fp32, q an integer
    nearest = dist == dist.min(axis=-1, keepdims=True)
    odd = (np.abs(qs) % 2 == 1)
    # among the nearest candidates prefer an even one (only differs at exact ties)
    pick = np.where(np.any(nearest & ~odd, axis=-1, keepdims=True), nearest & ~odd, nearest)
    return qs[np.argmax(pick, axis=-1)].astype(np.int64)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("clip", [1.0, 0.85, 0.6])
def test_brute_force_small_groups(bits, clip):
    """Every 4-element group over a 17-value grid (83,521 groups)."""
    grid = np.linspace(-2.0, 2.0, 17).astype(np.float32)  # dyadic steps of 1/4
    groups = np.array(list(itertools.product(grid, repeat=4)), dtype=np.float32)
    qmax = oracle.qmax_for_bits(bits)
    q, s = oracle.quant_act(groups, clip, bits, group=4)
    # independent per-group step from the definition, in Python scalars
    amax = np.array([max(abs(float(v)) for v in g) for g in groups], dtype=np.float32)
    base = (amax / np.float32(qmax)).astype(np.float32)
    step = (np.float32(clip) * base).astype(np.float32)
    np.testing.assert_array_equal(s[:, 0], step)
    nz = step > 0
    v = (groups[nz] / step[nz][:, None]).astype(np.float32)
    np.testing.assert_array_equal(q[nz].astype(np.int64), _brute_codes(v, qmax))
    assert np.all(q[~nz] == 0)


@pytest.mark.parametrize("bits", [4, 8])
def test_invariants_random_groups(bits):
    qmax = oracle.qmax_for_bits(bits)
    x = synth.with_outliers(synth.gaussian((64, 256), 11, bits), 3, 25.0, 12, bits)
    for clip in (1.0, 0.9, 0.7):
        q, s = oracle.quant_act(x, clip, bits)
        G = x.reshape(64, 8, 32)
        Q = q.reshape(64, 8, 32).astype(np.float64)
        # every non-zero group reaches +-qmax when c <= 1
        assert np.all(np.max(np.abs(Q), axis=2)[s > 0] == qmax)
        # reconstruction error: unclipped elements within s/2 (+ 1 fp32 ulp of x/s)
        rec = Q * s[:, :, None].astype(np.float64)
        err = np.abs(G.astype(np.float64) - rec)
        unclipped = np.abs(Q) < qmax
        bound = s[:, :, None].astype(np.float64) * (0.5 + 2.0 ** -20)
        assert np.all((err <= bound)[unclipped])
        # clipped error <= absmax (1 - c) + s/2
        amax = np.max(np.abs(G), axis=2, keepdims=True).astype(np.float64)
        cb = amax * (1 - clip) + bound + 1e-12
        assert np.all((err <= cb)[~unclipped])


# ---------------------------------------------------------------- roundings vs exact rationals

def _round_fraction_to_binary(fr: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Correctly rounded (nearest, ties to even) value of a rational in a binary
    format with mant_bits significand bits and minimum normal exponent emin."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def test_fp32_division_and_fp16_rounding_are_correctly_rounded():
    rng = synth.seeded_rng(synth.TEST, 31)
    a = (rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 4, 2000)).astype(np.float32)
    b = (np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-8, 2, 2000) + 1e-30).astype(np.float32)
    q = (a / b).astype(np.float32)
    for x, y, z in zip(a[:500], b[:500], q[:500]):
        exact = _round_fraction_to_binary(Fraction(float(x)) / Fraction(float(y)), 24, -126)
        assert Fraction(float(z)) == exact
    # fl16 as used for weight steps: normals, subnormals and exact ties
    vals = np.concatenate([
        (np.abs(rng.standard_normal(500)) * 10.0 ** rng.integers(-9, 4, 500)).astype(np.float32),
        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24 * 1.5, 2 ** -25, 65504.0], dtype=np.float32),
    ])
    h = vals.astype(np.float16)
    for v, hv in zip(vals, h):
        exact = _round_fraction_to_binary(Fraction(float(v)), 11, -14)
        assert Fraction(float(hv)) == exact


# ---------------------------------------------------------------- transform and fold

def test_transform_is_kronecker_product():
    rng = synth.seeded_rng(synth.TEST, 41)
    P1 = synth.haar_orthogonal(4, rng)
    P2 = synth.haar_orthogonal(6, rng)
    x = synth.gaussian((5, 24), 42)
    want = x.astype(np.float64) @ np.kron(P1.astype(np.float64), P2.astype(np.float64))
    np.testing.assert_allclose(oracle.kron_transform(x, P1, P2), want, rtol=0, atol=1e-13)
    # P1^T P1 = I for the generated factors (fp64 before fp32 rounding: fp32 error only)
    np.testing.assert_allclose(P1.astype(np.float64).T @ P1, np.eye(4), atol=1e-6)


def test_fold_is_inverse_kronecker_and_preserves_the_product():
    rng = synth.seeded_rng(synth.TEST, 43)
    P1 = synth.haar_orthogonal(4, rng)
    P2 = synth.haar_orthogonal(6, rng)
    W = synth.gaussian((7, 24), 44, scale=0.02)  # [N][K]
    P = np.kron(P1.astype(np.float64), P2.astype(np.float64))
    want = (np.linalg.inv(P) @ W.astype(np.float64).T).T
    got = oracle.fold_weights(W, P1, P2)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)
    # invariant: unquantized transform path reproduces x W (fp64; fp32 fold to 1e-6)
    x = synth.gaussian((5, 24), 45)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    y64 = oracle.kron_transform(x, P1, P2) @ got.T
    assert np.max(np.abs(y64 - ref)) <= 1e-12 * np.max(np.abs(ref))
    y32 = oracle.kron_transform(x, P1, P2) @ got.astype(np.float32).astype(np.float64).T
    assert np.max(np.abs(y32 - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_fold_with_non_orthogonal_factors_uses_the_inverse():
    rng = synth.seeded_rng(synth.TEST, 46)
    P1 = (np.eye(3) + 0.3 * rng.standard_normal((3, 3))).astype(np.float32)
    P2 = (np.eye(5) + 0.3 * rng.standard_normal((5, 5))).astype(np.float32)
    W = synth.gaussian((4, 15), 47)
    x = synth.gaussian((6, 15), 48)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    y = oracle.kron_transform(x, P1, P2) @ oracle.fold_weights(W, P1, P2).T
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_fold_at_block_shape_K2048():
    P1, P2 = synth.factors_for(synth.ouro_block_workload(), "qkv_in", 2048)
    W = synth.gaussian((3, 2048), 49, scale=0.02)
    x = synth.gaussian((4, 2048), 50)
    Wt = oracle.fold_weights(W, P1, P2).astype(np.float32)
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    y = oracle.kron_transform(x, P1, P2) @ Wt.astype(np.float64).T
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))


# ---------------------------------------------------------------- dots and rescale

def test_group_dots_brute_force_python_ints():
    rng = synth.seeded_rng(synth.TEST, 51)
    qa = rng.integers(-127, 128, size=(3, 96)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(4, 96)).astype(np.int8)
    d = oracle.group_dots(qa, qw)
    for m in range(3):
        for n in range(4):
            for j in range(3):
                s = 0
                for k in range(32 * j, 32 * j + 32):
                    s += int(qa[m, k]) * int(qw[n, k])
                assert int(d[m, n, j]) == s


@pytest.mark.parametrize("group_w", [32, 128])
def test_integer_path_equals_simulated_qdq(group_w):
    """Integer dots + rescale equals the quantize-dequantize product (the
    reproduction's simulated semantics, README "Protocol")."""
    x = synth.gaussian((8, 256), 52)
    w = synth.gaussian((16, 256), 53, scale=0.02)
    qw, sw = oracle.quant_weights(w, group_w)
    for bits in (4, 8):
        qa, sa = oracle.quant_act(x, 0.8, bits)
        y_int = oracle.rescale_dots(sa, oracle.group_dots(qa, qw), sw, group_w)
        y_qdq = oracle.qdq_linear(qa, sa, qw, sw, group_w)
        np.testing.assert_allclose(y_int, y_qdq, rtol=1e-12, atol=1e-15)


def test_rescale_uses_the_matching_weight_group():
    """A weight step placed in one g=128 group scales only the 4 activation
    groups it covers (catches an off-by-one or transposed group index)."""
    M, N, K = 2, 3, 256
    qa = np.ones((M, K), dtype=np.int8)
    qw = np.ones((N, K), dtype=np.int8)
    sa = np.ones((M, K // 32), dtype=np.float32)
    sw = np.zeros((N, 2), dtype=np.float16)
    sw[1, 1] = 2.0
    y = oracle.rescale_dots(sa, oracle.group_dots(qa, qw), sw, 128)
    np.testing.assert_array_equal(y[:, 1], 2.0 * 128)
    np.testing.assert_array_equal(y[:, 0], 0)
    sa2 = sa.copy()
    sa2[1, 5] = 3.0
    y2 = oracle.rescale_dots(sa2, oracle.group_dots(qa, qw), sw, 128)
    assert y2[1, 1] == 2.0 * (96 + 3 * 32) and y2[0, 1] == 2.0 * 128


# ---------------------------------------------------------------- special cases

def test_identity_transform_is_plain_group_rtn():
    x = synth.gaussian((4, 64), 54)
    np.testing.assert_array_equal(oracle.transformed_f32(x, None, None), x)
    I4 = np.eye(4, dtype=np.float32)
    I16 = np.eye(16, dtype=np.float32)
    np.testing.assert_array_equal(oracle.transformed_f32(x, I4, I16), x)


def test_per_token_arm_is_group_size_K():
    x = synth.gaussian((3, 64), 55)
    q, s = oracle.quant_act(x, 1.0, 4, group=64)
    amax = np.max(np.abs(x), axis=1)
    np.testing.assert_array_equal(s[:, 0], (amax / np.float32(7)).astype(np.float32))


def test_tail_groups_cover_only_real_elements():
    x = synth.gaussian((2, 80), 56)  # 2 full groups + a tail of 16
    q, s = oracle.quant_act(x, 1.0, 4)
    assert s.shape == (2, 3)
    tail_amax = np.max(np.abs(x[:, 64:]), axis=1)
    np.testing.assert_array_equal(s[:, 2], (tail_amax / np.float32(7)).astype(np.float32))
    w = synth.gaussian((3, 160), 57, scale=0.02)  # g=128: one group + a tail of 32
    qw, sw = oracle.quant_weights(w, 128)
    assert sw.shape == (3, 2)
    want = (np.max(np.abs(w[:, 128:]), axis=1) / np.float32(7)).astype(np.float32).astype(np.float16)
    np.testing.assert_array_equal(sw[:, 1], want)


def test_high_bit_activations_approach_the_plain_product():
    """bits_a -> 16 with clip 1: the layer output tends to x times the
    dequantized weights (a plain numpy product), within the activation RTN
    bound sum_k |s_a/2| |w_hat|."""
    wl = synth.tiny_workload()
    lin = wl.linears[0]
    P1, P2 = synth.factors_for(wl, "x", lin.K)
    W = synth.weights_for(wl, lin)
    Wt = oracle.fold_weights(W, P1, P2).astype(np.float32)
    qw, sw = oracle.quant_weights(Wt, 32)
    w_hat = qw.astype(np.float64) * np.repeat(sw.astype(np.float64), 32, axis=1)
    xs, _ = synth.activations_for(wl, "x", lin.K)
    x = xs[1]
    y, qa, sa = oracle.linear(x, P1, P2, 1.0, 16, qw, sw, 32)
    xt = oracle.kron_transform(x, P1, P2)
    ref = xt @ w_hat.T
    bound = (np.repeat(sa.astype(np.float64), 32, axis=1) * 0.5 + np.abs(xt) * 2.0 ** -23) @ np.abs(w_hat).T
    assert np.all(np.abs(y - ref) <= bound * 1.001 + 1e-12)
    assert np.max(np.abs(y - ref)) < 1e-3 * np.max(np.abs(ref))


def test_looped_forward_special_cases():
    wl = synth.tiny_workload()
    lin = wl.linears[0]
    P1, P2 = synth.factors_for(wl, "x", lin.K)
    W = oracle.fold_weights(synth.weights_for(wl, lin), P1, P2).astype(np.float32)
    qw, sw = oracle.quant_weights(W, 32)
    xs, _ = synth.activations_for(wl, "x", lin.K)
    clips = synth.clips_for(wl, "x")
    ys = oracle.looped_forward(xs, P1, P2, clips, 4, qw, sw, 32)
    # T = 1 is the single linear
    for t in range(wl.T):
        y1 = oracle.looped_forward(xs[t:t + 1], P1, P2, clips[t:t + 1], 4, qw, sw, 32)[0]
        np.testing.assert_array_equal(y1, ys[t])
    # equal (x_t, c_t) give equal y_t; a different clip changes the output
    same = oracle.looped_forward(np.stack([xs[0], xs[0]]), P1, P2, [clips[0], clips[0]], 4, qw, sw, 32)
    np.testing.assert_array_equal(same[0], same[1])
    diff = oracle.looped_forward(np.stack([xs[0], xs[0]]), P1, P2, [1.0, 0.7], 4, qw, sw, 32)
    assert not np.array_equal(diff[0], diff[1])
    # quantization error is small relative to the unquantized product
    ref = xs.astype(np.float64) @ synth.weights_for(wl, lin).astype(np.float64).T
    rel = np.max(np.abs(ys - ref)) / np.max(np.abs(ref))
    assert rel < 0.5


def test_weight_overflow_raises():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 7 * 65520.0
    with pytest.raises(OverflowError):
        oracle.quant_weights(w, 32)
    w[0, 0] = 7 * 65504.0
    oracle.quant_weights(w, 32)


def test_bf16_inputs_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    bits, wide = synth.round_to_bf16(x)
    np.testing.assert_array_equal(wide, np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0], dtype=np.float32))
    np.testing.assert_array_equal(bits, (wide.view(np.uint32) >> 16).astype(np.uint16))


# ---------------------------------------------------------------- Hadamard factors

def _fwht(x):
    """Walsh-Hadamard transform of each row by butterflies (natural order),
    unnormalized: x . H_K with H_K the Sylvester matrix of +-1."""
    y = np.array(x, dtype=np.float64)
    h = 1
    K = y.shape[1]
    while h < K:
        for i in range(0, K, 2 * h):
            a = y[:, i:i + h].copy()
            b = y[:, i + h:i + 2 * h].copy()
            y[:, i:i + h] = a + b
            y[:, i + h:i + 2 * h] = a - b
        h *= 2
    return y


@pytest.mark.parametrize("n1,n2", [(16, 16), (32, 64), (4, 8)])
def test_hadamard_factors_give_the_walsh_hadamard_transform(n1, n2):
    H1, H2 = synth.hadamard(n1), synth.hadamard(n2)
    np.testing.assert_allclose(H1.astype(np.float64) @ H1.T.astype(np.float64), np.eye(n1), atol=1e-6)
    x = synth.gaussian((5, n1 * n2), 170, n1, n2)
    got = oracle.kron_transform(x, H1, H2)
    # fp32 entries +-1/sqrt(n) carry the rounding of 1/sqrt(n) (exact for even log2 n)
    want = _fwht(x) / np.sqrt(n1 * n2)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


# ---------------------------------------------------------------- loop-dependent sets

def test_looped_forward_sets_reduces_to_shared_and_to_single_linears():
    wl = synth.tiny_workload()
    lin = wl.linears[0]
    xs, _ = synth.activations_for(wl, "x", lin.K)
    clips = synth.clips_for(wl, "x")
    P1, P2 = synth.factors_for(wl, "x", lin.K)
    Q1, Q2 = synth.hadamard(16), synth.hadamard(16)
    qw0, sw0 = oracle.quant_weights(synth.gaussian((lin.N, lin.K), 171, scale=0.02), 32)
    qw1, sw1 = oracle.quant_weights(synth.gaussian((lin.N, lin.K), 172, scale=0.02), 32)
    T = wl.T
    # one set for every loop and one bit width: the shared looped forward
    ys = oracle.looped_forward_sets(xs, [(P1, P2)], clips, [4] * T, [(qw0, sw0)], 32, [0] * T)
    np.testing.assert_array_equal(ys, oracle.looped_forward(xs, P1, P2, clips, 4, qw0, sw0, 32))
    # loop t on its own set and width: the single linear of that set
    sets, bits = [0, 1, 1, 0], [4, 8, 4, 8]
    ys = oracle.looped_forward_sets(xs, [(P1, P2), (Q1, Q2)], clips, bits, [(qw0, sw0), (qw1, sw1)], 32, sets)
    for t in range(T):
        F = [(P1, P2), (Q1, Q2)][sets[t]]
        W = [(qw0, sw0), (qw1, sw1)][sets[t]]
        y1, _, _ = oracle.linear(xs[t], F[0], F[1], float(clips[t]), bits[t], W[0], W[1], 32)
        np.testing.assert_array_equal(ys[t], y1)
    # the two sets differ, so the loops do too
    assert not np.array_equal(ys[0], oracle.looped_forward_sets(xs[:1], [(Q1, Q2)], clips[:1], [4], [(qw1, sw1)], 32, [0])[0])
    with pytest.raises(ValueError):
        oracle.looped_forward_sets(xs, [(P1, P2)], clips, [4] * T, [(qw0, sw0)], 32, [0] * (T - 1))


# ---------------------------------------------------------------- trajectory Hessian

def test_trajectory_hessian_brute_force_and_symmetry():
    xs = synth.gaussian((3, 5, 6), 190)
    H = oracle.trajectory_hessian(xs)
    B = np.zeros((6, 6))
    for t in range(3):                 # every outer product written out
        for m in range(5):
            for i in range(6):
                for j in range(6):
                    B[i, j] += float(xs[t, m, i]) * float(xs[t, m, j])
    np.testing.assert_allclose(H, B, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(H, H.T)
    assert np.linalg.eigvalsh(H)[0] > -1e-9           # positive semi-definite
    np.testing.assert_array_equal(oracle.trajectory_hessian(xs[0]), oracle.trajectory_hessian(xs[:1]))


def test_thresholded_rank_of_constructed_subspaces():
    # rows confined to an r-dimensional subspace give a rank-r Hessian; steps on
    # orthogonal subspaces add their ranks (the accumulated trajectory sees more)
    rng = synth.seeded_rng(synth.TEST, 191)
    K = 64
    Q, _ = np.linalg.qr(rng.standard_normal((K, K)))
    def step(cols, rows=40):
        Z = rng.standard_normal((rows, len(cols)))
        return Z @ Q[:, cols].T
    s0, s1 = step(list(range(0, 5))), step(list(range(5, 12)))
    assert oracle.thresholded_rank(oracle.trajectory_hessian(s0)) == 5
    assert oracle.thresholded_rank(oracle.trajectory_hessian(np.stack([s0, s1]))) == 12
    # directions below 1e-3 lambda_max do not count
    weak = s0 + 1e-3 * step(list(range(20, 30)))
    assert oracle.thresholded_rank(oracle.trajectory_hessian(weak)) == 5
    assert oracle.thresholded_rank(np.zeros((4, 4))) == 0


def test_per_token_hand_example():
    """One step per row ("The arms": rtn_w4a4_per_token), worked by hand.
    Row 0: absmax 7 over the whole row, so s = fl32(c * 7/7) = c.  Its second
    half only reaches 0.7, which a group of 32 would quantize on its own step
    0.1; per token it shares the row's step."""
    K = 64
    x = np.zeros((1, K), dtype=np.float32)
    x[0, :8] = [7.0, -3.5, 1.75, 0.0, 0.5, -0.25, 2.6, -7.0]
    x[0, 32:36] = [0.7, -0.5, 0.25, 0.6]
    qw = np.zeros((2, K), dtype=np.int8)
    qw[0, :8] = [1, 1, 1, 1, 1, 1, 1, 1]
    qw[1, 32:36] = [1, 2, -3, 7]
    sw = np.full((2, 2), np.float16(0.5))
    y, qa, sa = oracle.linear_per_token(x, None, None, 1.0, 4, qw, sw, 32)
    assert sa.shape == (1, 1) and sa[0, 0] == np.float32(1.0)
    # rint(x / 1), ties to even: -3.5 -> -4, 0.5 -> 0, -0.25 -> 0, 2.6 -> 3
    assert list(qa[0, :8]) == [7, -4, 2, 0, 0, 0, 3, -7]
    assert list(qa[0, 32:36]) == [1, 0, 0, 1]            # 0.7 -> 1, -0.5 -> 0, 0.25 -> 0, 0.6 -> 1
    # y = s_a * s_w * dot: row 0 of W: 0.5 * (7 - 4 + 2 + 3 - 7) = 0.5; row 1: 0.5 * (1 + 0 + 0 + 7) = 4
    np.testing.assert_array_equal(y, [[0.5, 4.0]])
    # clip 0.5: s = 0.5; x / s = 14, -7, 3.5, 0, 1, -0.5, 5.2, -14 -> 7, -7, 4, 0, 1, 0, 5, -7
    _, qa2, sa2 = oracle.linear_per_token(x, None, None, 0.5, 4, qw, sw, 32)
    assert sa2[0, 0] == np.float32(0.5)
    assert list(qa2[0, :8]) == [7, -7, 4, 0, 1, 0, 5, -7]
    # group-32 quantizes the second half on its own step 0.1 instead
    _, qg, sg = oracle.linear(x, None, None, 1.0, 4, qw, sw, 32)
    assert sg[0, 1] == np.float32(np.float32(0.7) / np.float32(7.0))
    assert list(qg[0, 32:36]) != list(qa[0, 32:36])


def test_per_token_equals_groups_when_group_maxima_agree_and_the_fold_form():
    """Rows whose 32-groups all have the same absmax give identical codes and
    steps per token and per group; and the per-token y equals the group fold
    with the row's step repeated in every group slot (the layout the GPU GEMM
    consumes), up to fp64 summation order."""
    rng = synth.seeded_rng(synth.TEST, 192)
    M, K, N = 5, 128, 7
    x = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
    x[:, ::32] = np.float32(3.0)                  # every group's absmax is 3
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    sw = rng.uniform(0.01, 0.1, size=(N, K // 32)).astype(np.float16)
    yt, qt, st = oracle.linear_per_token(x, None, None, 0.8, 4, qw, sw, 32)
    yg, qg, sg = oracle.linear(x, None, None, 0.8, 4, qw, sw, 32)
    np.testing.assert_array_equal(qt, qg)
    np.testing.assert_array_equal(np.repeat(st, K // 32, axis=1), sg)
    np.testing.assert_allclose(yt, yg, rtol=1e-12, atol=1e-12)
    # general rows: the fold with repeated steps
    x = synth.with_outliers(synth.gaussian((M, K), 193), 3, 20.0, 194)
    yt, qt, st = oracle.linear_per_token(x, None, None, 0.9, 8, qw, sw, 128)
    folded = oracle.rescale_dots(np.repeat(st, K // 32, axis=1), oracle.group_dots(qt, qw), sw, 128)
    np.testing.assert_allclose(yt, folded, rtol=1e-12, atol=1e-9)


def test_recurrent_adapter_with_a_scaled_identity_weight():
    """W = [7 I | 0]: the weight group holding the diagonal has step
    fl16(7/7) = 1 and code 7, every other group is zero, so the linear returns
    7 times the dequantized state, and the
    recurrence is s_{t+1} = 7 * s_t^ with s_t^ the Eq.(4) group RTN of s_t (the
    e half meets zero weights).  Written out per element with plain numpy:
    step per 32-group fl32(c * fl32(absmax / 7)), code rint(fl32(s / step))."""
    M, N = 3, 64
    s0 = synth.gaussian((M, N), 195)
    e = synth.gaussian((M, N), 196, scale=5.0)
    W = np.zeros((N, 2 * N), dtype=np.float32)
    W[:, :N] = 7.0 * np.eye(N, dtype=np.float32)
    qw, sw = oracle.quant_weights(W, 32)
    want_sw = np.zeros((N, 2 * N // 32), dtype=np.float16)
    want_sw[np.arange(N), np.arange(N) // 32] = 1.0   # the diagonal's group; all-zero groups have step 0
    np.testing.assert_array_equal(sw, want_sw)
    np.testing.assert_array_equal(qw[:, :N], 7 * np.eye(N))
    clips = [1.0, 0.8, 0.9]
    got = oracle.recurrent_adapter(s0, e, None, None, clips, 4, qw, sw, 32)
    s = s0.astype(np.float32)
    for t, c in enumerate(clips):
        nxt = np.empty_like(s)
        for m in range(M):
            for g in range(N // 32):
                blk = s[m, 32 * g:32 * g + 32]
                step = np.float32(np.float32(c) * np.float32(np.float32(np.max(np.abs(blk))) / np.float32(7)))
                q = np.clip(np.rint(np.float32(blk / step)), -7, 7)
                nxt[m, 32 * g:32 * g + 32] = 7.0 * (q * np.float64(step))
        s = nxt.astype(np.float32)
        np.testing.assert_array_equal(got[t], s)
    # T = 1 is one linear on cat(s_0, e)
    y1, _, _ = oracle.linear(np.concatenate([s0, e], axis=1), None, None, 1.0, 4, qw, sw, 32)
    np.testing.assert_array_equal(got[0], y1.astype(np.float32))
