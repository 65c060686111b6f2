"""Pins of the oracle's CTA functions (the loop-transition adapter of
"paper_specification.yaml", ``loopq_components.cta``, Section 4.3, Eq.(7);
``cta_rank: 8``) against hand-computed values, a library rounding and the
algebra of the map, not against the formula retyped."""

import numpy as np
import pytest
import torch

import oracle
from bit_ptq_looped_amd import synth


def test_round_bf16_ties_and_subnormals_by_hand():
    # bf16 keeps 8 significant bits: the spacing just above 1 is 2^-7
    assert oracle.round_bf16(1 + 2.0 ** -8) == 1.0                  # tie, even mantissa kept
    assert oracle.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6     # tie, rounds up to even
    assert oracle.round_bf16(1 + 2.0 ** -8 + 2.0 ** -30) == 1 + 2.0 ** -7
    assert oracle.round_bf16(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    assert oracle.round_bf16(0.0) == 0.0
    # below 2^-126 the spacing is 2^-133
    assert oracle.round_bf16(2.0 ** -130 + 2.0 ** -140) == 2.0 ** -130
    assert oracle.round_bf16(2.0 ** -133 * 2.5) == 2.0 ** -133 * 2


def test_round_bf16_matches_torch_on_fp32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even: on values that
    # are exact in fp32 the one rounding must agree
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(v.astype(np.float64)), want)


def test_identity_parameters_leave_rows_unchanged():
    rng = np.random.default_rng(1)
    K, r = 96, 8
    h = rng.standard_normal((5, K))
    U, V = rng.standard_normal((K, r)), rng.standard_normal((K, r))
    out = oracle.cta_transition(h, U, V, np.ones(K), np.zeros(K), 0.0)
    np.testing.assert_array_equal(out, h)


def test_rank_one_by_hand():
    # U = e_1, V = e_0: V^T h picks h_0 = 3, U puts eta * 3 = 6 on element 1
    h = np.array([[3.0, 5.0, 7.0, 11.0]])
    U = np.array([[0.0], [1.0], [0.0], [0.0]])
    V = np.array([[1.0], [0.0], [0.0], [0.0]])
    out = oracle.cta_transition(h, U, V, np.ones(4), np.zeros(4), 2.0)
    np.testing.assert_array_equal(out, [[3.0, 11.0, 7.0, 11.0]])
    # with the affine part: a = (1, 2, 1, 1), b = (0, 0, 0.5, 0)
    out = oracle.cta_transition(h, U, V, np.array([1.0, 2.0, 1.0, 1.0]), np.array([0.0, 0.0, 0.5, 0.0]), 2.0)
    np.testing.assert_array_equal(out, [[3.0, 16.0, 7.5, 11.0]])


def test_rank_two_fixes_the_roles_of_U_and_V():
    # V reads elements 1 and 3 (5 and 11), U writes them to elements 0 and 2;
    # swapping U and V would read 3 and 7 and write to 1 and 3
    h = np.array([[3.0, 5.0, 7.0, 11.0]])
    U = np.array([[1.0, 0.0], [0.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    V = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 0.0], [0.0, 1.0]])
    out = oracle.cta_transition(h, U, V, np.ones(4), np.zeros(4), 1.0)
    np.testing.assert_array_equal(out, [[8.0, 5.0, 18.0, 11.0]])


def test_zero_gate_is_the_affine_map_by_hand():
    h = np.array([[1.0, 2.0, 3.0]])
    rng = np.random.default_rng(2)
    out = oracle.cta_transition(h, rng.standard_normal((3, 8)), rng.standard_normal((3, 8)),
                                np.full(3, 2.0), np.full(3, -1.0), 0.0)
    np.testing.assert_array_equal(out, [[1.0, 3.0, 5.0]])


def test_shared_orthonormal_pair_scales_its_span_only():
    # U = V = Q with orthonormal columns: U V^T is the projector on span(Q), so
    # the map is h + eta P h: (1 + eta) h on the span, h on its complement
    rng = np.random.default_rng(3)
    K, r, eta = 64, 8, 0.5
    Q, _ = np.linalg.qr(rng.standard_normal((K, r)))
    inside = rng.standard_normal((4, r)) @ Q.T
    g = rng.standard_normal((4, K))
    outside = g - (g @ Q) @ Q.T
    ones, zeros = np.ones(K), np.zeros(K)
    np.testing.assert_allclose(oracle.cta_transition(inside, Q, Q, ones, zeros, eta), 1.5 * inside, atol=1e-12)
    np.testing.assert_allclose(oracle.cta_transition(outside, Q, Q, ones, zeros, eta), outside, atol=1e-12)


def test_loop_inputs_take_transition_t_minus_1_and_leave_loop_0():
    # a_0 = 2, a_1 = 3 on small integers: loop 1 reads 2 x_1, loop 2 reads 3 x_2
    rng = np.random.default_rng(4)
    K = 32
    xs = rng.integers(-8, 9, (3, 2, K)).astype(np.float64)
    U = rng.standard_normal((K, 8))
    V = rng.standard_normal((K, 8))
    a = np.stack([np.full(K, 2.0), np.full(K, 3.0)])
    b = np.zeros((2, K))
    for state in ("bf16", "fp32"):
        got = oracle.cta_loop_inputs(xs, U, V, a, b, [0.0, 0.0], state)
        np.testing.assert_array_equal(got[0], xs[0])
        np.testing.assert_array_equal(got[1], 2 * xs[1])
        np.testing.assert_array_equal(got[2], 3 * xs[2])


def test_bf16_state_is_rounded_once_to_bf16():
    # 1 + 2^-8 is not a bf16 value: the stored state rounds it (tie -> 1)
    K = 32
    xs = np.ones((2, 1, K))
    b = np.full((1, K), 2.0 ** -8)
    got = oracle.cta_loop_inputs(xs, np.zeros((K, 8)), np.zeros((K, 8)), np.ones((1, K)), b, [0.0], "bf16")
    np.testing.assert_array_equal(got[1], np.ones((1, K)))
    got = oracle.cta_loop_inputs(xs, np.zeros((K, 8)), np.zeros((K, 8)), np.ones((1, K)), b, [0.0], "fp32")
    np.testing.assert_array_equal(got[1], np.full((1, K), 1 + 2.0 ** -8))


@pytest.mark.parametrize("state", ["bf16", "fp32"])
def test_identity_cta_forward_is_the_plain_looped_forward(state):
    wl = synth.tiny_workload()
    lin = wl.linears[0]
    K = lin.K
    P1, P2 = synth.factors_for(wl, "x", K)
    W = synth.weights_for(wl, lin)
    xs, _ = synth.activations_for(wl, "x", K)
    if state == "bf16":  # a bf16 state holds bf16 values
        xs = oracle.round_bf16(xs)
    clips = synth.clips_for(wl, "x")
    qw, sw = oracle.quant_weights(oracle.fold_weights(W, P1, P2).astype(np.float32), 32)
    T = xs.shape[0]
    rng = np.random.default_rng(5)
    U, V = rng.standard_normal((K, 8)), rng.standard_normal((K, 8))
    a, b, eta = np.ones((T - 1, K)), np.zeros((T - 1, K)), np.zeros(T - 1)
    got = oracle.looped_forward_cta(xs, P1, P2, clips, 4, qw, sw, 32, U, V, a, b, eta, state)
    want = oracle.looped_forward(xs, P1, P2, clips, 4, qw, sw, 32)
    np.testing.assert_array_equal(got, want)
