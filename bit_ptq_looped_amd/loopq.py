"""Python binding of libloopq (the C ABI in include/loopq.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C function of the same name, and raises :class:`LoopQError` on a non-zero
status.  There is no fallback: if the library is missing or fails to load,
:func:`load` raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libloopq.so")

LOOPQ_ABI_VERSION = 2
LOOPQ_OK = 0
LOOPQ_ERR_INVALID_ARG = -1
LOOPQ_ERR_UNSUPPORTED = -2
LOOPQ_ERR_ALIGNMENT = -3
LOOPQ_ERR_RANGE = -4
LOOPQ_ERR_HIP = -5
LOOPQ_ERR_WORKSPACE = -6
LOOPQ_ERR_SINGULAR = -7

LOOPQ_F32, LOOPQ_BF16 = 0, 1
LOOPQ_SCHED_AUTO, LOOPQ_SCHED_LOOP_SEQUENTIAL, LOOPQ_SCHED_WEIGHT_STATIONARY = 0, 1, 2
LOOPQ_OP_LINEAR, LOOPQ_OP_LOOPED_FORWARD, LOOPQ_OP_FOLD, LOOPQ_OP_LOOPED_FORWARD_EX = 1, 2, 3, 4
LOOPQ_OP_HESSIAN, LOOPQ_OP_QUANT_PER_TOKEN, LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN = 5, 6, 7
LOOPQ_OP_RECURRENT_ADAPTER, LOOPQ_OP_LOOPED_FORWARD_CTA, LOOPQ_OP_LOOPED_FORWARD_HESSIAN = 8, 9, 10
LOOPQ_KERNEL_QUANT_TRANSFORM, LOOPQ_KERNEL_QUANT_PLAIN, LOOPQ_KERNEL_GEMM, LOOPQ_KERNEL_DECODE = 0, 1, 2, 3
LOOPQ_KERNEL_HESSIAN, LOOPQ_KERNEL_QUANT_TOKEN, LOOPQ_KERNEL_CTA = 4, 5, 6

# every entry point of include/loopq.h with its ctypes signature
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_ZP = ctypes.POINTER(ctypes.c_size_t)
SIGNATURES = {
    "loopq_abi_version": ([], _I),
    "loopq_status_string": ([_I], ctypes.c_char_p),
    "loopq_packed_weight_bytes": ([_I, _I, _I, _ZP, _ZP], _I),
    "loopq_workspace_bytes": ([_I, _I, _I, _I, _I, _I, _ZP], _I),
    "loopq_fold_weights": ([_P, _I, _I, _P, _I, _P, _I, _P, _P, _Z, _P], _I),
    "loopq_pack_weights": ([_P, _I, _I, _I, _P, _P, _P], _I),
    "loopq_quant_act": ([_P, _I, _I, _I, _P, _I, _P, _I, _F, _I, _P, _P, _P, _P], _I),
    "loopq_w4a4_linear": ([_P, _I, _I, _I, _I, _P, _I, _P, _I, _F, _I, _P, _P, _I, _P, _P, _Z, _P], _I),
    "loopq_looped_forward": ([_P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _I,
                              _P, _Z, _P], _I),
    "loopq_looped_forward_ex": ([_P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P, _I, _P, _P, _P,
                                 _P, _P, _Z, _P], _I),
    "loopq_gemm_codes": ([_P, _P, _I, _I, _I, _P, _P, _I, _I, _P, _P, _Z, _P], _I),
    "loopq_w4a4_linear_noalloc": ([_P, _I, _I, _I, _I, _P, _I, _P, _I, _F, _I, _P, _P, _I, _P, _P], _I),
    "loopq_noalloc_scratch_bytes": ([], _Z),
    "loopq_export_weights": ([_P, _P, _I, _I, _I, _P, _P, _P], _I),
    "loopq_group_dots": ([_P, _I, _I, _I, _I, _P, _P, _P, _Z, _P], _I),
    "loopq_export_weight_codes": ([_P, _I, _I, _I, _P, _P], _I),
    "loopq_export_act_codes": ([_P, _Z, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "loopq_hessian_accumulate": ([_P, _I, _I, _P, _P, _Z, _P], _I),
    "loopq_recurrent_adapter": ([_P, _P, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _P, _Z, _P], _I),
    "loopq_quant_act_per_token": ([_P, _I, _I, _I, _P, _I, _P, _I, _F, _I, _P, _P, _P, _P, _Z, _P], _I),
    "loopq_looped_forward_per_token": ([_P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _P, _Z,
                                        _P], _I),
    "loopq_looped_forward_hessian": ([_P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _I,
                                      _P, _P, _Z, _P], _I),
    "loopq_cta_apply": ([_P, _I, _I, _I, _P, _P, _I, _P, _P, _F, _P, _P], _I),
    "loopq_looped_forward_cta": ([_P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _I,
                                  _P, _P, _I, _P, _P, _P, _P, _Z, _P], _I),
    "loopq_timing_enable": ([_I], _I),
    "loopq_timing_read": ([_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)], _I),
    "loopq_timing_reset": ([], _I),
}

_lib = None


class LoopQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().loopq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def load(path: Optional[str] = None):
    """Load the shared library once; raise if it is missing or mismatched."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m bit_ptq_looped_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.loopq_abi_version() != LOOPQ_ABI_VERSION:
        raise RuntimeError("libloopq ABI version mismatch")
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != LOOPQ_OK:
        raise LoopQError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    return t.data_ptr()


_torch = None
_raw_stream = None


def _torch_mod():
    global _torch, _raw_stream
    if _torch is None:
        import torch
        # the current stream's handle as an int: torch's raw getter costs a
        # tenth of building a Stream object, which matters for few-row calls
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _torch = torch
    return _torch


def _stream(stream) -> Optional[int]:
    if stream is None:
        torch = _torch_mod()
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(x) -> int:
    torch = _torch_mod()
    if x.dtype == torch.float32:
        return LOOPQ_F32
    if x.dtype == torch.bfloat16:
        return LOOPQ_BF16
    raise ValueError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _factor_args(P1, P2):
    if P1 is None and P2 is None:
        return None, 0, None, 0
    return _ptr(P1), int(P1.shape[0]), _ptr(P2), int(P2.shape[0])


# ----------------------------------------------------------------- host-only calls

def loopq_abi_version() -> int:
    return load().loopq_abi_version()


def loopq_status_string(status: int) -> str:
    return load().loopq_status_string(status).decode()


def loopq_packed_weight_bytes(K: int, N: int, group_w: int):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().loopq_packed_weight_bytes(K, N, group_w, ctypes.byref(c), ctypes.byref(s)),
           "loopq_packed_weight_bytes")
    return c.value, s.value


def loopq_workspace_bytes(op: int, T: int, M: int, K: int, N: int, bits_a: int) -> int:
    b = ctypes.c_size_t()
    _check(load().loopq_workspace_bytes(op, T, M, K, N, bits_a, ctypes.byref(b)), "loopq_workspace_bytes")
    return b.value


# ----------------------------------------------------------------- device calls

def loopq_fold_weights(w, P1, P2, w_folded, workspace, stream=None):
    N, K = w.shape
    _check(load().loopq_fold_weights(_ptr(w), K, N, _ptr(P1), int(P1.shape[0]), _ptr(P2),
                                     int(P2.shape[0]), _ptr(w_folded), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_fold_weights")


def loopq_pack_weights(w_folded, group_w: int, w_codes, w_scales, stream=None):
    N, K = w_folded.shape
    _check(load().loopq_pack_weights(_ptr(w_folded), K, N, group_w, _ptr(w_codes), _ptr(w_scales),
                                     _stream(stream)), "loopq_pack_weights")


def loopq_quant_act(x, P1, P2, clip: float, bits_a: int, codes, scales, xt_out=None, stream=None):
    M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    _check(load().loopq_quant_act(_ptr(x), _dtype_code(x), M, K, p1, n1, p2, n2, float(clip), bits_a,
                                  _ptr(codes), _ptr(scales), _ptr(xt_out), _stream(stream)),
           "loopq_quant_act")


def loopq_w4a4_linear(x, P1, P2, clip: float, bits_a: int, w_codes, w_scales, group_w: int, N: int,
                      y, workspace, stream=None):
    M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    _check(load().loopq_w4a4_linear(_ptr(x), _dtype_code(x), M, K, N, p1, n1, p2, n2, float(clip),
                                    bits_a, _ptr(w_codes), _ptr(w_scales), group_w, _ptr(y),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "loopq_w4a4_linear")


def loopq_w4a4_linear_noalloc(x, P1, P2, clip: float, bits_a: int, w_codes, w_scales, group_w: int, N: int,
                              y, stream=None):
    """loopq_w4a4_linear on the library's fixed scratch (no workspace)."""
    M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    _check(load().loopq_w4a4_linear_noalloc(_ptr(x), _dtype_code(x), M, K, N, p1, n1, p2, n2, float(clip), bits_a,
                                            _ptr(w_codes), _ptr(w_scales), group_w, _ptr(y), _stream(stream)),
           "loopq_w4a4_linear_noalloc")


def loopq_noalloc_scratch_bytes() -> int:
    return int(load().loopq_noalloc_scratch_bytes())


def loopq_looped_forward(x, P1, P2, clips: Sequence[float], bits_a: int, w_codes, w_scales,
                         group_w: int, N: int, y, schedule: int, workspace, stream=None):
    T, M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    _check(load().loopq_looped_forward(_ptr(x), _dtype_code(x), T, M, K, N, p1, n1, p2, n2,
                                       ctypes.cast(c, ctypes.c_void_p), bits_a, _ptr(w_codes),
                                       _ptr(w_scales), group_w, _ptr(y), schedule, _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_looped_forward")


def loopq_looped_forward_hessian(x, P1, P2, clips: Sequence[float], bits_a: int, w_codes, w_scales,
                                 group_w: int, N: int, y, schedule: int, H, workspace, stream=None):
    """loopq_looped_forward that also accumulates H += x~^T x~ over all loops."""
    T, M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    _check(load().loopq_looped_forward_hessian(_ptr(x), _dtype_code(x), T, M, K, N, p1, n1, p2, n2,
                                               ctypes.cast(c, ctypes.c_void_p), bits_a, _ptr(w_codes),
                                               _ptr(w_scales), group_w, _ptr(y), schedule, _ptr(H), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_looped_forward_hessian")


def loopq_cta_apply(h, U, V, a, b, eta: float, out, stream=None):
    """One CTA transition on the rows of h [M][K] into out (may be h)."""
    M, K = h.shape
    _check(load().loopq_cta_apply(_ptr(h), _dtype_code(h), M, K, _ptr(U), _ptr(V), int(U.shape[1]), _ptr(a),
                                  _ptr(b), float(eta), _ptr(out), _stream(stream)),
           "loopq_cta_apply")


def loopq_looped_forward_cta(x, P1, P2, clips: Sequence[float], bits_a: int, w_codes, w_scales,
                             group_w: int, N: int, y, schedule: int, U, V, a_sets, b_sets,
                             etas: Sequence[float], workspace, stream=None):
    """loopq_looped_forward with CTA transition t - 1 applied to loop t >= 1."""
    T, M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    ev = [float(v) for v in etas][: max(T - 1, 0)]
    e = (ctypes.c_float * max(len(ev), 1))(*ev)
    rank = int(U.shape[1]) if U is not None else 0
    _check(load().loopq_looped_forward_cta(_ptr(x), _dtype_code(x), T, M, K, N, p1, n1, p2, n2,
                                           ctypes.cast(c, ctypes.c_void_p), bits_a, _ptr(w_codes),
                                           _ptr(w_scales), group_w, _ptr(y), schedule, _ptr(U), _ptr(V), rank,
                                           _ptr(a_sets), _ptr(b_sets), ctypes.cast(e, ctypes.c_void_p),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)),
           "loopq_looped_forward_cta")


def loopq_looped_forward_ex(x, factor_sets, clips: Sequence[float], bits: Sequence[int], weight_sets,
                            group_w: int, N: int, y, sets: Sequence[int], workspace, stream=None):
    """factor_sets: a list of (P1, P2) device tensors per set, or None (no
    transform); weight_sets: a list of (w_codes, w_scales) per set; sets, bits
    and clips: one entry per loop."""
    T, M, K = x.shape
    nsets = len(weight_sets)
    VP = ctypes.c_void_p * nsets
    if factor_sets is None:
        p1 = p2 = None
        n1 = n2 = 0
    else:
        if len(factor_sets) != nsets:
            raise ValueError("one factor pair per weight set")
        p1 = VP(*[_ptr(f[0]) for f in factor_sets])
        p2 = VP(*[_ptr(f[1]) for f in factor_sets])
        n1, n2 = int(factor_sets[0][0].shape[0]), int(factor_sets[0][1].shape[0])
    wc = VP(*[_ptr(w[0]) for w in weight_sets])
    wsc = VP(*[_ptr(w[1]) for w in weight_sets])
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    st = (ctypes.c_int32 * T)(*[int(v) for v in sets])
    bt = (ctypes.c_int32 * T)(*[int(v) for v in bits])
    as_p = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
    _check(load().loopq_looped_forward_ex(_ptr(x), _dtype_code(x), T, M, K, N, nsets, as_p(p1), n1, as_p(p2),
                                          n2, as_p(wc), as_p(wsc), group_w, as_p(st), as_p(bt), as_p(c),
                                          _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _stream(stream)), "loopq_looped_forward_ex")


def loopq_gemm_codes(a_codes, a_scales, w_codes, w_scales, group_w: int, N: int, y, workspace,
                     bits_a: int = 4, stream=None):
    M, K = a_codes.shape
    _check(load().loopq_gemm_codes(_ptr(a_codes), _ptr(a_scales), M, K, N, _ptr(w_codes),
                                   _ptr(w_scales), group_w, bits_a, _ptr(y), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_gemm_codes")


def loopq_export_weights(w_codes, w_scales, K: int, N: int, group_w: int, codes, scales, stream=None):
    _check(load().loopq_export_weights(_ptr(w_codes), _ptr(w_scales), K, N, group_w, _ptr(codes),
                                       _ptr(scales), _stream(stream)), "loopq_export_weights")


def loopq_export_weight_codes(w_codes, K: int, N: int, group_w: int, codes, stream=None):
    _check(load().loopq_export_weight_codes(_ptr(w_codes), K, N, group_w, _ptr(codes), _stream(stream)),
           "loopq_export_weight_codes")


def loopq_export_act_codes(workspace, op: int, T: int, M: int, K: int, N: int, bits_a: int, schedule: int,
                           codes, scales, stream=None):
    """The codes [T*M][K] int8 and steps [T*M][K/32] fp32 the last forward call
    of this op and shape left in ``workspace``."""
    _check(load().loopq_export_act_codes(_ptr(workspace), workspace.numel() * workspace.element_size(), op, T,
                                         M, K, N, bits_a, schedule, _ptr(codes), _ptr(scales), _stream(stream)),
           "loopq_export_act_codes")


def loopq_group_dots(a_codes, w_codes, N: int, dots, workspace, bits_a: int = 4, stream=None):
    M, K = a_codes.shape
    _check(load().loopq_group_dots(_ptr(a_codes), M, K, N, bits_a, _ptr(w_codes), _ptr(dots), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_group_dots")


def loopq_quant_act_per_token(x, P1, P2, clip: float, bits_a: int, codes, scales, xt_out=None,
                              workspace=None, stream=None):
    M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().loopq_quant_act_per_token(_ptr(x), _dtype_code(x), M, K, p1, n1, p2, n2, float(clip), bits_a,
                                            _ptr(codes), _ptr(scales), _ptr(xt_out), _ptr(workspace), nbytes,
                                            _stream(stream)), "loopq_quant_act_per_token")


def loopq_looped_forward_per_token(x, P1, P2, clips: Sequence[float], bits_a: int, w_codes, w_scales,
                                   group_w: int, N: int, y, workspace, stream=None):
    """x [T][M][K] (or [M][K] for one loop), one clip per loop."""
    if x.dim() == 2:
        x = x.unsqueeze(0)
    T, M, K = x.shape
    p1, n1, p2, n2 = _factor_args(P1, P2)
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    _check(load().loopq_looped_forward_per_token(_ptr(x), _dtype_code(x), T, M, K, N, p1, n1, p2, n2,
                                                 ctypes.cast(c, ctypes.c_void_p), bits_a, _ptr(w_codes),
                                                 _ptr(w_scales), group_w, _ptr(y), _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_looped_forward_per_token")


def loopq_recurrent_adapter(s0, e, P1, P2, clips: Sequence[float], bits_a: int, w_codes, w_scales,
                            group_w: int, y, workspace, stream=None):
    """s0, e fp32 [M][N]; y fp32 [T][M][N] receives s_1 .. s_T."""
    M, N = s0.shape
    T = len(clips)
    p1, n1, p2, n2 = _factor_args(P1, P2)
    c = (ctypes.c_float * T)(*[float(v) for v in clips])
    _check(load().loopq_recurrent_adapter(_ptr(s0), _ptr(e), T, M, N, p1, n1, p2, n2,
                                          ctypes.cast(c, ctypes.c_void_p), bits_a, _ptr(w_codes), _ptr(w_scales),
                                          group_w, _ptr(y), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream)),
           "loopq_recurrent_adapter")


def loopq_hessian_accumulate(xt, H, workspace=None, stream=None):
    """H += xt^T xt; xt fp32 [rows][K], H fp32 [K][K], both on the device."""
    rows, K = xt.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().loopq_hessian_accumulate(_ptr(xt), rows, K, _ptr(H), _ptr(workspace), nbytes,
                                           _stream(stream)), "loopq_hessian_accumulate")


def loopq_timing_enable(on: bool) -> None:
    _check(load().loopq_timing_enable(1 if on else 0), "loopq_timing_enable")


def loopq_timing_reset() -> None:
    _check(load().loopq_timing_reset(), "loopq_timing_reset")


def loopq_timing_read(n: int = 7):
    """Per kernel id: (total milliseconds, launches) since the last read."""
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load().loopq_timing_read(n, ms, cnt), "loopq_timing_read")
    return [(ms[k], cnt[k]) for k in range(n)]


# ----------------------------------------------------------------- buffer helpers

def empty_packed_weights(K: int, N: int, group_w: int, device="cuda"):
    """Uninitialized device buffers sized for loopq_pack_weights."""
    import torch
    cb, sb = loopq_packed_weight_bytes(K, N, group_w)
    return (torch.empty(cb, dtype=torch.uint8, device=device),
            torch.empty(sb, dtype=torch.uint8, device=device))


def empty_workspace(op: int, T: int, M: int, K: int, N: int, bits_a: int, device="cuda"):
    import torch
    n = loopq_workspace_bytes(op, T, M, K, N, bits_a)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)
