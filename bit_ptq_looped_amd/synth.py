"""Seeded synthetic workloads for the looped quantized linear.

This module only draws inputs: random orthogonal factors, weights,
activations with outlier channels and loop drift, and per-loop clips.  It
holds none of the method's arithmetic (no transform, fold, quantization or
product), so the tests can hand the same arrays to the HIP library and to the
CPU oracle.

Every array comes from numpy's PCG64 seeded with ``SeedSequence([workload,
tensor, layer, loop, ...])`` so a case is reproducible from its key alone.
Activations that the workloads declare as bf16 are rounded to bf16 here
(round to nearest even) and returned both as raw bf16 bits (for the device)
and widened to fp32 (exact, for the oracle).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# workload ids used in the seed keys
TINY, OURO_BLOCK, DECODE, HUGINN, LARGE_PREFILL, TEST = 1, 2, 3, 4, 5, 9
# tensor ids used in the seed keys
T_X, T_W, T_P1, T_P2, T_CLIP, T_OUTLIER, T_AUX = 1, 2, 3, 4, 5, 6, 7


def seeded_rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def haar_orthogonal(n: int, rng: np.random.Generator) -> np.ndarray:
    """Random orthogonal n x n matrix (QR of a Gaussian matrix with the signs of
    R's diagonal moved into Q), drawn in fp64 and stored as fp32."""
    a = rng.standard_normal((n, n))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def hadamard(n: int) -> np.ndarray:
    """Normalized Sylvester-Hadamard matrix of order n (a power of two), entries
    +-1/sqrt(n), as fp32: the Hadamard choice of a Kronecker factor ("Quantizing
    Looped Transformers", rotation ablation, Table 14).  H_a kron H_b is H_ab."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return (h / np.sqrt(n)).astype(np.float32)


def round_to_bf16(x: np.ndarray):
    """Round fp32 values to bf16 (nearest, ties to even).

    Returns ``(bits uint16, widened float32)``; widening bf16 to fp32 is exact.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) & 0xFFFF0000).astype(np.uint32)
    bits = (r >> 16).astype(np.uint16)
    return bits, r.view(np.float32)


@dataclass
class Linear:
    """One weight matrix of a looped block and the quantized input it reads."""
    name: str
    K: int
    N: int
    act: str  # name of the quantized input tensor (one clip per input and loop)


@dataclass
class Workload:
    name: str
    wid: int
    M: int
    T: int
    bits_a: int
    group_w: int
    linears: list
    factors: dict = field(default_factory=dict)  # K -> (n1, n2); empty = no transform
    layers: int = 1


def ouro_like_linears(hidden: int, inter: int):
    """q/k/v/o and an MLP up/down pair of a transformer block; q, k and v read
    the same quantized input (they share one clip per loop)."""
    return [
        Linear("q", hidden, hidden, "qkv_in"), Linear("k", hidden, hidden, "qkv_in"),
        Linear("v", hidden, hidden, "qkv_in"), Linear("o", hidden, hidden, "o_in"),
        Linear("up", hidden, inter, "up_in"), Linear("down", inter, hidden, "down_in"),
    ]


def tiny_workload():
    return Workload("tiny looped linear M=16 K=256 N=128 T=4", TINY, M=16, T=4, bits_a=4,
                    group_w=32, linears=[Linear("w", 256, 128, "x")], factors={256: (16, 16)})


def ouro_block_workload(bits_a: int = 4, M: int = 1024, T: int = 4, layers: int = 1):
    return Workload(f"Ouro-1.4B-like looped block M={M} hidden 2048 MLP 5632 T={T} W4A{bits_a}",
                    OURO_BLOCK, M=M, T=T, bits_a=bits_a, group_w=32,
                    linears=ouro_like_linears(2048, 5632),
                    factors={2048: (32, 64), 5632: (64, 88)}, layers=layers)


def decode_workload(M: int, T: int = 4, layers: int = 24, bits_a: int = 4):
    w = ouro_block_workload(bits_a=bits_a, M=M, T=T, layers=layers)
    w.name = f"decode Ouro-1.4B-like {layers} layers M={M} T={T} W4A{bits_a}"
    w.wid = DECODE
    return w


def huginn_workload(M: int = 2048, T: int = 32):
    return Workload(f"Huginn-like recurrence M={M} T={T} W4(g128)A8", HUGINN, M=M, T=T, bits_a=8,
                    group_w=128,
                    linears=[Linear("adapter", 10560, 5280, "adapter_in"),
                             Linear("wqkv", 5280, 15840, "core_in"),
                             Linear("mlp_proj", 17920, 5280, "proj_in")],
                    factors={})


def large_prefill_workload(T: int = 4, M: int = 8192, layers: int = 48):
    return Workload(f"2.6B-like looped stack M={M} hidden 2560 MLP 6912 T={T} W4A4", LARGE_PREFILL,
                    M=M, T=T, bits_a=4, group_w=32, linears=ouro_like_linears(2560, 6912),
                    factors={2560: (40, 64), 6912: (64, 108)}, layers=layers)


# ---------------------------------------------------------------------------
# drawing tensors
# ---------------------------------------------------------------------------

def factors_for(wl: Workload, act: str, K: int, layer: int = 0):
    """(P1, P2) for one quantized input, shared across loops; None if the
    workload has no transform for this K."""
    if K not in wl.factors:
        return None, None
    n1, n2 = wl.factors[K]
    aid = _act_id(act)
    P1 = haar_orthogonal(n1, seeded_rng(wl.wid, T_P1, layer, aid))
    P2 = haar_orthogonal(n2, seeded_rng(wl.wid, T_P2, layer, aid))
    return P1, P2


def weights_for(wl: Workload, lin: Linear, layer: int = 0) -> np.ndarray:
    """fp32 weights stored [N][K], N(0, 0.02^2)."""
    rng = seeded_rng(wl.wid, T_W, layer, _lin_id(lin.name))
    return (rng.standard_normal((lin.N, lin.K), dtype=np.float32) * np.float32(0.02))


def clips_for(wl: Workload, act: str, layer: int = 0) -> np.ndarray:
    """Per-loop LAS clips for one quantized input, fp32 [T]."""
    if wl.wid == TINY:
        lo, hi = 0.7, 1.0
    elif wl.wid == HUGINN:
        return np.ones(wl.T, dtype=np.float32)
    else:
        lo, hi = 0.6, 1.0
    rng = seeded_rng(wl.wid, T_CLIP, layer, _act_id(act))
    return rng.uniform(lo, hi, size=wl.T).astype(np.float32)


def activations_for(wl: Workload, act: str, K: int, layer: int = 0, rows: int | None = None):
    """Loop inputs ``[T][M][K]`` for one quantized input.

    Returns ``(device_array, fp32_array)``: for bf16 workloads the device
    array holds bf16 bits (uint16) and the fp32 array is their exact widening;
    for the tiny workload both are the same fp32 array.
    """
    M = wl.M if rows is None else rows
    T = wl.T
    aid = _act_id(act)
    if wl.wid == TINY:
        rng = seeded_rng(wl.wid, T_X, layer, aid)
        x0 = rng.standard_normal((M, K))
        ch = seeded_rng(wl.wid, T_OUTLIER, layer, aid).choice(K, size=2, replace=False)
        x0[:, ch] *= 20.0
        xs = np.stack([(1.0 + 0.25 * t) * x0 + 0.1 * t for t in range(T)]).astype(np.float32)
        return xs, xs
    if wl.wid == HUGINN:
        xs = _huginn_states(wl, act, K, M, layer)
    elif wl.wid == LARGE_PREFILL:
        n_out = int(round(0.005 * K))
        ch = seeded_rng(wl.wid, T_OUTLIER, layer, aid).choice(K, size=n_out, replace=False)
        xs = np.empty((T, M, K), dtype=np.float32)
        for t in range(T):
            x = seeded_rng(wl.wid, T_X, layer, aid, t).standard_normal((M, K), dtype=np.float32)
            x[:, ch] *= np.float32(30.0)
            xs[t] = x + np.float32(0.1 * t)
    else:  # Ouro-like block and decode
        n_out = int(round(0.01 * K))
        ch = seeded_rng(wl.wid, T_OUTLIER, layer, aid).choice(K, size=n_out, replace=False)
        xs = np.empty((T, M, K), dtype=np.float32)
        for t in range(T):
            rng = seeded_rng(wl.wid, T_X, layer, aid, t)
            x = rng.standard_normal((M, K), dtype=np.float32)
            x[:, ch] = rng.standard_t(3.0, size=(M, n_out)).astype(np.float32)
            xs[t] = x * np.float32(1.0 + 0.25 * t)
    bits, widened = round_to_bf16(xs)
    return bits, widened


def _huginn_states(wl: Workload, act: str, K: int, M: int, layer: int) -> np.ndarray:
    """Recurrent states x_{t+1} = 0.9 x_t + 0.1 xi_t; the adapter input adds a
    rank-43 drifting component Z_t B / sqrt(43)."""
    T = wl.T
    aid = _act_id(act)
    rng = seeded_rng(wl.wid, T_X, layer, aid)
    xs = np.empty((T, M, K), dtype=np.float32)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if act == "adapter_in":
        rank = 43
        B = seeded_rng(wl.wid, T_AUX, layer, aid).standard_normal((rank, K), dtype=np.float32)
        Z = rng.standard_normal((M, rank), dtype=np.float32)
    for t in range(T):
        if act == "adapter_in":
            xs[t] = (Z @ B) / np.float32(np.sqrt(43.0)) + np.float32(0.1) * x
            Z = np.float32(0.9) * Z + np.float32(0.1) * rng.standard_normal((M, rank), dtype=np.float32)
        else:
            xs[t] = x
        x = np.float32(0.9) * x + np.float32(0.1) * rng.standard_normal((M, K), dtype=np.float32)
    return xs


_ACTS = ["x", "qkv_in", "o_in", "up_in", "down_in", "adapter_in", "core_in", "proj_in"]
_LINS = ["w", "q", "k", "v", "o", "up", "down", "adapter", "wqkv", "mlp_proj"]


def _act_id(name: str) -> int:
    return _ACTS.index(name) + 1


def _lin_id(name: str) -> int:
    return _LINS.index(name) + 1


# ---------------------------------------------------------------------------
# small generic cases for tests
# ---------------------------------------------------------------------------

def gaussian(shape, *key, scale: float = 1.0) -> np.ndarray:
    return (seeded_rng(TEST, *key).standard_normal(shape) * scale).astype(np.float32)


def uniform(shape, lo: float, hi: float, *key) -> np.ndarray:
    return seeded_rng(TEST, *key).uniform(lo, hi, size=shape).astype(np.float32)


def with_outliers(x: np.ndarray, n_channels: int, factor: float, *key) -> np.ndarray:
    x = np.array(x, dtype=np.float32, copy=True)
    ch = seeded_rng(TEST, *key).choice(x.shape[-1], size=n_channels, replace=False)
    x[..., ch] *= np.float32(factor)
    return x
