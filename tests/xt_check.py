"""Parity reading for the Kronecker transform, shared by the GPU tests.

The pages fix no precision for the transform: "paper_specification.yaml" lists
the Kronecker factorization details among its underspecified items, and its
runs simulate quantization on a bf16 base model.  The kernels form
x~ = vec_r(P1^T X P2) with fp32 products and fp32 accumulation, so parity has
two parts:

1. the kernel's x~ (the ``xt_out`` dump of ``loopq_quant_act``, the values it
   quantized) lies element by element within the fp32-class bound
       |x~_gpu - x~_64| <= 8 (n1 + n2) 2^-24 (|P1|^T |X| |P2|)
   of the oracle's fp64 transform;
2. codes and steps are bit-exact, and y within 1e-4, against the oracle
   applied to that dump (no transform on the oracle side).

A row's x~ depends only on the row and the fixed sequence of MFMA steps, so
the dump of ``loopq_quant_act`` is bitwise the x~ every other entry point
quantizes for the same rows and factors.
"""

import numpy as np
import torch

import oracle

XT_BOUND_FACTOR = 8.0


def xt_bound(x32, P1, P2):
    """8 (n1 + n2) 2^-24 |P1|^T |X| |P2| per element, fp64, [rows][K]."""
    n1, n2 = P1.shape[0], P2.shape[0]
    ax = np.abs(np.asarray(x32, dtype=np.float64))
    mag = oracle.kron_transform(ax, np.abs(P1), np.abs(P2))
    return XT_BOUND_FACTOR * (n1 + n2) * 2.0 ** -24 * mag


def check_xt(dump, x32, P1, P2):
    """Assert part 1 for the rows of ``dump`` (fp32 [rows][K]) whose inputs are
    ``x32``; returns the largest |error| / bound seen."""
    want = oracle.kron_transform(x32, P1, P2)
    err = np.abs(np.asarray(dump, dtype=np.float64) - want)
    bound = xt_bound(x32, P1, P2)
    ratio = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), f"x~ outside the fp32-class bound (max error/bound {ratio:.3f})"
    return ratio


def gpu_xt(lq, xdev, x32, P1, P2):
    """The kernel's x~ for the rows of ``xdev`` ([rows][K] on the device, fp32
    or bf16; ``x32`` its fp32 values on the host), checked against the bound.
    With no transform it is x itself."""
    x32 = np.asarray(x32, dtype=np.float32).reshape(xdev.shape[0], -1)
    if P1 is None:
        return x32
    rows, K = xdev.shape
    codes = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.float32, device="cuda")
    xt = torch.empty((rows, K), dtype=torch.float32, device="cuda")
    lq.loopq_quant_act(xdev, torch.from_numpy(np.ascontiguousarray(P1)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(P2)).cuda(), 1.0, 4, codes, scales, xt)
    torch.cuda.synchronize()
    dump = xt.cpu().numpy()
    check_xt(dump, x32, P1, P2)
    return dump


# ---------------------------------------------------------------------------
# Parity reading for the trajectory Hessian (H += x~^T x~).  The kernel
# multiplies on the bf16 matrix cores: each fp32 x~ value is split into three
# bf16 planes whose sum is the value exactly (hi = the value truncated to
# bf16, mid = the remainder truncated, lo = the rest), and each product
# x~_ri x~_rj is taken as the six plane products of order <= 2, each exact in
# fp32; the three dropped ones (mid lo, lo mid, lo lo) are below
# 2 * 2^-7 * 2^-14 + 2^-28 < 2^-20 of |x~_ri x~_rj|, and the kept ones sum to
# at most (1 + 2^-6) |x~_ri x~_rj|.  They are added in fp32: six additions per
# row, at most one per 64-row piece of a tile split across work groups, and
# the final addition to H, so an element of H0 + sum_r x~_r^T x~_r lies within
#   gamma(6 rows + ceil(rows / 64) + 2) ((1 + 2^-6) |x~|^T |x~| + |H0|) + 2^-20 |x~|^T |x~|
# of the exact value, gamma(n) = n u / (1 - n u), u = 2^-24.  Chained calls
# add their bounds.
# ---------------------------------------------------------------------------
HESS_U = 2.0 ** -24


def hessian_bound(rows, mag_x, mag_h0=0.0):
    """The element-wise bound above for one call over `rows` rows, with
    mag_x = (|x~|^T |x~|)_ij and mag_h0 = |H0_ij| (scalars or arrays)."""
    n = 6 * rows + -(-rows // 64) + 2
    gamma = n * HESS_U / (1.0 - n * HESS_U)
    return gamma * ((1.0 + 2.0 ** -6) * mag_x + mag_h0) + 2.0 ** -20 * mag_x
