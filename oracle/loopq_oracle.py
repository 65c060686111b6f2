"""Plain CPU oracle for the looped W4A4 / W4A8 group-quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link this module; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code, table or helper with the HIP path.

It is deliberately slow and literal: numpy arrays, one step of the method per
function, fp64 wherever the pages do not fix a precision.  Sources (titles of
the pages the method is described on):

* "LoopQ 4-bit quantization of Ouro-1.4B -- raw artifacts" (README of a LoopQ
  reproduction): sections "The arms" and "Protocol" -- RTN with activations in
  groups of 32, random orthogonal Kronecker transforms with LAS clip 1.0 for
  the untrained LoopQ arm, one set of 24 layers applied four times to every
  token, quantization simulated as quantize-dequantize.
* "paper_specification.yaml" of the same reproduction: ``lq1_quantization``
  (Eq.(4) ``Q_a(x; c) = c * clip(round(x / c), q_min, q_max)``, RTN, W4 with A4
  or A8, group-wise, group size 32), ``loopq_components`` (shared transformed
  backbone with an invertible transform folded into both sides; LAS: one
  clipping scalar per module and loop), ``implementation_status`` lq2 (clips
  multiply dynamic token/group absmax scales) and lq3 (shared Kronecker
  transform folded into the weights by its exact inverse transpose before
  quantization), and the list of
  ``paper_underspecified_items``.
* "Quantizing Looped Transformers: Feedback Exposure and Calibration
  Blindness": Figure 3 and Tables 2 and 6 -- grouped INT4 weights with g=128.

Readings taken where the pages leave a point open (each also listed in the
design notes):

* integer bounds: symmetric ``[-(2^(b-1)-1), 2^(b-1)-1]`` -- [-7, 7] for 4 bit,
  [-127, 127] for 8 bit;
* ties: round half to even (``np.rint``);
* scale: the Eq.(4) step is ``c * absmax / qmax`` over the group, computed as
  ``fl32(c * fl32(absmax / qmax))``; activation steps stay fp32, weight steps
  are ``fl16(fl32(absmax / 7))`` and weight codes are computed with that
  fp16-rounded step; division is correctly rounded fp32 division, never a
  multiply by a reciprocal; an all-zero (or underflowed) group has step 0 and
  codes 0;
* groups: consecutive elements along K (the reduction axis) of the flat
  row-major index; the last group may be short and its absmax covers only its
  real elements;
* transform: ``x~ = x . (P1 (x) P2) = vec_r(P1^T X P2)`` with ``X`` the
  row-major ``n1 x n2`` reshape of a row, and the folded weight (stored one
  output column per row, ``[N][K]``) ``w~_n = vec_r(P1^-1 W_n P2^-T)``;
* the transformed activation is formed in fp64 and rounded once to fp32
  before it is quantized.
* CTA ("paper_specification.yaml", ``loopq_components.cta``, Section 4.3,
  Eq.(7), which the pages do not print; ``experiment_hyperparameters``
  ``cta_rank: 8``; "The arms": CTA at exact identity in the untrained arm): at
  the transition into loop t (t >= 1) a row h of the state becomes
  ``a_{t-1} * h + b_{t-1} + eta_{t-1} * U (V^T h)`` -- an elementwise affine
  map plus a scalar-gated low-rank term, U and V (``[K][r]``) shared by every
  transition, a, b (``[K]``) and eta per transition; identity is a = 1, b = 0,
  eta = 0.  It is formed in fp64 and stored in the state's type (bf16: round
  to nearest, ties to even; fp32: one fp32 rounding) before loop t reads it.

Functions with no pin against anything but themselves: none -- every function
here is pinned by ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import numpy as np

GROUP_A = 32  # activation group size ("lq1_quantization": granularity, group_size 32)


def qmax_for_bits(bits: int) -> int:
    """Largest code of the symmetric signed b-bit grid (reading of the
    unspecified ``integer_bounds`` item): 7 for 4 bit, 127 for 8 bit."""
    if bits < 2:
        raise ValueError("bits must be >= 2")
    return (1 << (bits - 1)) - 1


def _group_bounds(K: int, g: int):
    """Half-open K ranges of consecutive groups of size g; the last one may be
    short (reading of ``group_axis_and_tail_layout``)."""
    return [(j0, min(K, j0 + g)) for j0 in range(0, K, g)]


# --------------------------------------------------------------------------
# a0 -- transform and weight fold (spec: "shared_transformed_backbone";
#        implementation_status lq3: a Kronecker transform whose exact
#        inverse transpose is folded into the unquantized weights)
# --------------------------------------------------------------------------

def kron_transform(x: np.ndarray, P1: np.ndarray, P2: np.ndarray) -> np.ndarray:
    """Transformed activations ``x~[m] = vec_r(P1^T X_m P2)`` in fp64.

    ``x`` is ``[M][K]`` (any float dtype, widened exactly to fp64), ``P1`` is
    ``n1 x n1`` and ``P2`` is ``n2 x n2`` with ``K = n1 * n2``.  This is the row
    vector ``x`` times the Kronecker product ``P1 (x) P2``.
    """
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    n1, n2 = P1.shape[0], P2.shape[0]
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if n1 * n2 != K:
        raise ValueError("n1 * n2 must equal K")
    X = x.reshape(M, n1, n2)
    out = np.matmul(np.matmul(P1.T[None, :, :], X), P2[None, :, :])
    return out.reshape(M, K)


def fold_weights(w: np.ndarray, P1: np.ndarray, P2: np.ndarray) -> np.ndarray:
    """Folded weights ``W~ = (P1 (x) P2)^-1 W`` in fp64, stored ``[N][K]``.

    Row n of the storage is output column n of the math-convention ``K x N``
    weight, so ``w~_n = vec_r(P1^-1 W_n P2^-T)``.  The inverses are the exact
    fp64 inverses of the given factors (for orthogonal factors they equal the
    transposes up to rounding).  Round the result once to fp32 to obtain the
    weights the quantizer sees.
    """
    P1 = np.asarray(P1, dtype=np.float64)
    P2 = np.asarray(P2, dtype=np.float64)
    n1, n2 = P1.shape[0], P2.shape[0]
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    if n1 * n2 != K:
        raise ValueError("n1 * n2 must equal K")
    P1i = np.linalg.inv(P1)
    P2i = np.linalg.inv(P2)
    Wn = w.reshape(N, n1, n2)
    out = np.matmul(np.matmul(P1i[None, :, :], Wn), P2i.T[None, :, :])
    return out.reshape(N, K)


# --------------------------------------------------------------------------
# a1 -- weight quantization (Eq.(4) with clip 1, group-wise, W4)
# --------------------------------------------------------------------------

def quant_weights(w32: np.ndarray, group_w: int):
    """RTN INT4 codes and fp16 steps for fp32 weights stored ``[N][K]``.

    Per output column n and K-group j (size ``group_w``, last group short):
    ``s32 = fl32(absmax / 7)``, ``s16 = fl16(s32)``; if ``s16 == 0`` the codes
    are 0, else ``q = clamp(rint(fl32(w / fl32(s16))), -7, 7)``.

    Returns ``(codes int8 [N][K], scales float16 [N][ceil(K/group_w)])``.
    Raises ``OverflowError`` if a step does not fit fp16.
    """
    w32 = np.asarray(w32)
    if w32.dtype != np.float32:
        raise TypeError("weights must be float32")
    N, K = w32.shape
    groups = _group_bounds(K, group_w)
    codes = np.zeros((N, K), dtype=np.int8)
    scales = np.zeros((N, len(groups)), dtype=np.float16)
    qmax = np.float32(7)
    for j, (k0, k1) in enumerate(groups):
        blk = w32[:, k0:k1]
        amax = np.max(np.abs(blk), axis=1)                      # exact
        s32 = (amax / qmax).astype(np.float32)                   # fl32 division
        with np.errstate(over="ignore"):
            s16 = s32.astype(np.float16)                         # RNE to binary16
        if not np.all(np.isfinite(s16)):
            raise OverflowError("weight group step overflows fp16")
        sdiv = s16.astype(np.float32)
        safe = np.where(sdiv > 0, sdiv, np.float32(1))
        q = np.rint((blk / safe[:, None]).astype(np.float32))    # fl32 division, ties to even
        q = np.clip(q, -7, 7)
        q[sdiv == 0, :] = 0
        codes[:, k0:k1] = q.astype(np.int8)
        scales[:, j] = s16
    return codes, scales


# --------------------------------------------------------------------------
# a3, a4 -- activation step and RTN codes (Eq.(4); LAS clip c_{t,l})
# --------------------------------------------------------------------------

def quant_act(xt32: np.ndarray, clip: float, bits: int, group: int = GROUP_A):
    """Eq.(4) group RTN of fp32 transformed activations ``[M][K]``.

    Per row m and group j of ``group`` consecutive elements:
    ``base = fl32(absmax / qmax)``, ``s = fl32(c * base)`` with the LAS clip
    ``c``; ``s == 0`` gives codes 0 and step 0, otherwise
    ``q = clamp(rint(fl32(x / s)), -qmax, qmax)``.

    Returns ``(codes int8/int16 [M][K], steps float32 [M][ceil(K/group)])``.
    """
    xt32 = np.asarray(xt32)
    if xt32.dtype != np.float32:
        raise TypeError("transformed activations must be float32")
    qmax = qmax_for_bits(bits)
    c = np.float32(clip)
    M, K = xt32.shape
    groups = _group_bounds(K, group)
    code_dtype = np.int8 if qmax <= 127 else np.int32
    codes = np.zeros((M, K), dtype=code_dtype)
    steps = np.zeros((M, len(groups)), dtype=np.float32)
    for j, (k0, k1) in enumerate(groups):
        blk = xt32[:, k0:k1]
        amax = np.max(np.abs(blk), axis=1)                       # exact
        base = (amax / np.float32(qmax)).astype(np.float32)       # fl32 division
        s = (c * base).astype(np.float32)                         # fl32 product
        safe = np.where(s > 0, s, np.float32(1))
        q = np.rint((blk / safe[:, None]).astype(np.float32))     # fl32 division, ties to even
        q = np.clip(q, -qmax, qmax)
        q[s == 0, :] = 0
        codes[:, k0:k1] = q.astype(code_dtype)
        steps[:, j] = s
    return codes, steps


# --------------------------------------------------------------------------
# a5 -- integer group dots and the per-group rescale
# --------------------------------------------------------------------------

def group_dots(qa: np.ndarray, qw: np.ndarray, group: int = GROUP_A) -> np.ndarray:
    """Exact per-group integer dot products ``d[m, n, j] = sum_{k in j} qa[m,k] qw[n,k]``.

    ``qa`` is ``[M][K]``, ``qw`` is ``[N][K]``; returns int64 ``[M][N][G]``.
    """
    qa = np.asarray(qa).astype(np.int64)
    qw = np.asarray(qw).astype(np.int64)
    M, K = qa.shape
    N, K2 = qw.shape
    if K != K2:
        raise ValueError("K mismatch")
    groups = _group_bounds(K, group)
    d = np.zeros((M, N, len(groups)), dtype=np.int64)
    for j, (k0, k1) in enumerate(groups):
        d[:, :, j] = qa[:, k0:k1] @ qw[:, k0:k1].T
    return d


def rescale_dots(sa: np.ndarray, d: np.ndarray, sw16: np.ndarray, group_w: int,
                 group_a: int = GROUP_A) -> np.ndarray:
    """``y[m, n] = sum_j sa[m, j] * sw[n, (group_a * j) // group_w] * d[m, n, j]`` in fp64.

    Activation group j covers K indices ``[group_a*j, group_a*(j+1))``; it lies
    inside weight group ``(group_a*j) // group_w`` because ``group_w`` is a
    multiple of ``group_a``.
    """
    if group_w % group_a != 0:
        raise ValueError("group_w must be a multiple of the activation group")
    sa = np.asarray(sa, dtype=np.float64)
    sw = np.asarray(sw16).astype(np.float64)
    M, N, G = d.shape
    y = np.zeros((M, N), dtype=np.float64)
    for j in range(G):
        jw = (group_a * j) // group_w
        y += (sa[:, j][:, None] * sw[:, jw][None, :]) * d[:, :, j].astype(np.float64)
    return y


def qdq_linear(qa, sa, qw, sw16, group_w: int, group_a: int = GROUP_A) -> np.ndarray:
    """The simulated (quantize-dequantize) product the reproduction evaluates:
    dequantize both operands in fp64 and multiply.  Must equal
    :func:`rescale_dots` of :func:`group_dots` up to fp64 summation order."""
    qa = np.asarray(qa, dtype=np.float64)
    qw = np.asarray(qw, dtype=np.float64)
    M, K = qa.shape
    N = qw.shape[0]
    ka = np.arange(K) // group_a
    kw = np.arange(K) // group_w
    a_hat = qa * np.asarray(sa, dtype=np.float64)[:, ka]
    w_hat = qw * np.asarray(sw16).astype(np.float64)[:, kw]
    return a_hat @ w_hat.T


# --------------------------------------------------------------------------
# a2..a6 -- one linear and the loop over t
# --------------------------------------------------------------------------

def transformed_f32(x: np.ndarray, P1, P2) -> np.ndarray:
    """The fp32 activations the quantizer sees: ``fl32(vec_r(P1^T X P2))``
    from an fp64 transform, or ``x`` itself when there is no transform."""
    if P1 is None and P2 is None:
        return np.asarray(x, dtype=np.float32)
    return kron_transform(x, P1, P2).astype(np.float32)


def linear(x, P1, P2, clip: float, bits: int, qw, sw16, group_w: int):
    """One quantized linear: transform, Eq.(4) activation RTN, integer group
    dots, fp64 rescale.  Returns ``(y fp64 [M][N], codes, steps)``."""
    xt32 = transformed_f32(x, P1, P2)
    qa, sa = quant_act(xt32, clip, bits)
    d = group_dots(qa, qw)
    y = rescale_dots(sa, d, sw16, group_w)
    return y, qa, sa


def linear_per_token(x, P1, P2, clip: float, bits: int, qw, sw16, group_w: int):
    """The per-token arm: the same RTN with one activation step per token
    ("LoopQ 4-bit quantization of Ouro-1.4B -- raw artifacts", "The arms":
    ``rtn_w4a4_per_token``).  Eq.(4) over the whole row (one group of K),
    weights as for :func:`linear` (group-wise), and the dequantized product.
    Returns ``(y fp64 [M][N], codes, steps [M][1])``."""
    xt32 = transformed_f32(x, P1, P2)
    K = xt32.shape[1]
    qa, sa = quant_act(xt32, clip, bits, group=K)
    y = qdq_linear(qa, sa, qw, sw16, group_w, group_a=K)
    return y, qa, sa


def recurrent_adapter(s0, e, P1, P2, clips, bits: int, qw, sw16, group_w: int) -> np.ndarray:
    """A dependent recurrence through one quantized linear.  In the Huginn
    recurrence loop ("Quantizing Looped Transformers", Figure 4) the adapter
    reads the state concatenated with the embedding, ``cat(s_t, e)``, and its
    output feeds the recurrence directly, with no skip connection around it.
    Leaving out the recurrent blocks between two adapter calls gives
    ``s_{t+1} = fl32(linear(cat(s_t, e)))`` with loop t's clip.
    ``s0`` and ``e`` are ``[M][N]``, the weight ``[N][2N]``; returns the states
    ``s_1 .. s_T`` as fp32 ``[T][M][N]`` (the state is kept in fp32 between
    loops, as a device would store it)."""
    s = np.asarray(s0, dtype=np.float32)
    e = np.asarray(e, dtype=np.float32)
    out = []
    for c in clips:
        x = np.concatenate([s, e], axis=1)
        y, _, _ = linear(x, P1, P2, float(c), bits, qw, sw16, group_w)
        s = y.astype(np.float32)
        out.append(s)
    return np.stack(out)


def looped_forward(xs, P1, P2, clips, bits: int, qw, sw16, group_w: int) -> np.ndarray:
    """The same quantized weights applied at every loop t with the loop's own
    LAS clip ``clips[t]`` (spec ``las``: one clip per module and loop).
    ``xs`` is ``[T][M][K]``; returns fp64 ``[T][M][N]``."""
    xs = np.asarray(xs)
    T = xs.shape[0]
    if len(clips) != T:
        raise ValueError("one clip per loop")
    return np.stack([linear(xs[t], P1, P2, float(clips[t]), bits, qw, sw16, group_w)[0]
                     for t in range(T)])


def looped_forward_sets(xs, factor_sets, clips, bits, weight_sets, group_w: int, sets) -> np.ndarray:
    """The loop with loop-dependent pieces: loop t uses transform and weights of
    set ``sets[t]`` and activation bit width ``bits[t]``.

    SLT ("paper_specification.yaml", ``loopq_components.slt``, Section 4.2,
    Eqs. (5)-(6)): the transform and weight groups SLT picks vary with the loop,
    the rest stay shared.  A per-loop activation bit width is the output of a loop-wise
    precision allocation ("Quantisation errors can keep returning inside a
    looped model", "Three components address three sources of mismatch").
    ``factor_sets`` is a list of ``(P1, P2)`` (or ``(None, None)``),
    ``weight_sets`` a list of ``(qw, sw16)``; returns fp64 ``[T][M][N]``."""
    xs = np.asarray(xs)
    T = xs.shape[0]
    if not (len(clips) == len(bits) == len(sets) == T):
        raise ValueError("one clip, bit width and set per loop")
    out = []
    for t in range(T):
        P1, P2 = factor_sets[sets[t]]
        qw, sw = weight_sets[sets[t]]
        out.append(linear(xs[t], P1, P2, float(clips[t]), int(bits[t]), qw, sw, group_w)[0])
    return np.stack(out)



# --------------------------------------------------------------------------
# CTA: the loop-transition adapter ("paper_specification.yaml",
#      loopq_components.cta, Section 4.3, Eq.(7); cta_rank 8)
# --------------------------------------------------------------------------

def round_bf16(v) -> np.ndarray:
    """``v`` (fp64) rounded to the nearest bfloat16 value (8 significant bits,
    fp32's exponent range), ties to even; returned as fp64.  Values past the
    largest finite bf16 are not handled (the adapted states stay far below)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                      # v = m 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2^-126 the spacing stays 2^-133
    ulp = np.ldexp(1.0, e - 8)
    return np.rint(v / ulp) * ulp           # v / ulp is exact (power of two)


def cta_transition(h, U, V, a, b, eta) -> np.ndarray:
    """One loop transition of CTA on the rows of ``h`` ``[M][K]``:
    ``a * h + b + eta * U (V^T h)`` per row, in fp64.  ``U`` and ``V`` are
    ``[K][r]`` (the shared low-rank pair), ``a`` and ``b`` ``[K]`` and ``eta`` a
    scalar (this transition's parameters)."""
    h = np.asarray(h, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    z = h @ V                               # [M][r]: V^T h of every row
    return np.asarray(a, dtype=np.float64) * h + np.asarray(b, dtype=np.float64) + float(eta) * (z @ U.T)


def cta_loop_inputs(xs, U, V, a_sets, b_sets, etas, state: str) -> np.ndarray:
    """The inputs the loops read with CTA at every transition: loop 0 reads
    ``xs[0]``; loop t >= 1 reads transition t-1 applied to ``xs[t]``, stored
    as ``state`` ("bf16" or "fp32").  ``a_sets``/``b_sets`` are ``[T-1][K]``,
    ``etas`` ``[T-1]``; returns fp64 ``[T][M][K]``."""
    xs = np.asarray(xs, dtype=np.float64)
    T = xs.shape[0]
    if not (len(a_sets) >= T - 1 and len(b_sets) >= T - 1 and len(etas) >= T - 1):
        raise ValueError("one set of transition parameters per transition")
    store = {"bf16": round_bf16, "fp32": lambda v: v.astype(np.float32).astype(np.float64)}[state]
    out = [xs[0]]
    for t in range(1, T):
        out.append(store(cta_transition(xs[t], U, V, a_sets[t - 1], b_sets[t - 1], etas[t - 1])))
    return np.stack(out)


def looped_forward_cta(xs, P1, P2, clips, bits: int, qw, sw16, group_w: int, U, V, a_sets, b_sets, etas,
                       state: str) -> np.ndarray:
    """:func:`looped_forward` with CTA at the loop transitions: loop t >= 1
    quantizes the adapted state of :func:`cta_loop_inputs`."""
    return looped_forward(cta_loop_inputs(xs, U, V, a_sets, b_sets, etas, state), P1, P2, clips, bits, qw,
                          sw16, group_w)


# --------------------------------------------------------------------------
# next: trajectory Hessian ("Quantizing Looped Transformers": the GPTQ
#       Hessian accumulated across recurrence steps; Table 1, thresholded rank
#       at 1e-3 lambda_max)
# --------------------------------------------------------------------------

def trajectory_hessian(xts) -> np.ndarray:
    """``H = sum_t X_t^T X_t`` in fp64 over the steps' (transformed) activations
    ``xts`` ``[T][M][K]`` (or one ``[M][K]`` step): the Hessian a GPTQ step uses,
    built from every recurrence step instead of step 0 only."""
    xts = np.asarray(xts, dtype=np.float64)
    if xts.ndim == 2:
        xts = xts[None]
    K = xts.shape[2]
    H = np.zeros((K, K))
    for x in xts:
        H += x.T @ x
    return H


def thresholded_rank(H, rel: float = 1e-3) -> int:
    """Number of eigenvalues of the symmetric PSD ``H`` above ``rel * lambda_max``
    (Table 1's rank measure)."""
    ev = np.linalg.eigvalsh(np.asarray(H, dtype=np.float64))
    lmax = ev[-1]
    if lmax <= 0:
        return 0
    return int(np.count_nonzero(ev > rel * lmax))
