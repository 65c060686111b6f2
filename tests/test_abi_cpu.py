"""The C ABI library loads without a GPU, exports every symbol include/loopq.h
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from bit_ptq_looped_amd import loopq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loopq.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int32_t|size_t|const char\*)\s+(loopq_\w+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(loopq.LIB_PATH):
        from bit_ptq_looped_amd import build
        build.build(verbose=False)
    return loopq.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) == 27
    for n in names:
        assert hasattr(lib, n), n
        assert n in loopq.SIGNATURES, n
    assert set(loopq.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert loopq.loopq_abi_version() == loopq.LOOPQ_ABI_VERSION
    for st in range(0, -8, -1):
        assert loopq.loopq_status_string(st) != "unknown status"
    assert loopq.loopq_status_string(-99) == "unknown status"


def test_packed_sizes(lib):
    cb, sb = loopq.loopq_packed_weight_bytes(2048, 5632, 32)
    assert cb == 5632 * 2048 // 2 and sb == 5632 * 64 * 2
    cb, sb = loopq.loopq_packed_weight_bytes(10560, 5280, 128)
    assert cb == 5280 * 10560 // 2 and sb == 5280 * 83 * 2  # 82 full groups + a tail of 64
    cb, sb = loopq.loopq_packed_weight_bytes(64, 40, 32)  # ragged N padded to 64 columns
    assert cb == 64 * 64 // 2 and sb == 64 * 2 * 2
    with pytest.raises(loopq.LoopQError) as e:
        loopq.loopq_packed_weight_bytes(33, 8, 32)
    assert e.value.status == loopq.LOOPQ_ERR_UNSUPPORTED
    with pytest.raises(loopq.LoopQError) as e:
        loopq.loopq_packed_weight_bytes(64, 8, 64)
    assert e.value.status == loopq.LOOPQ_ERR_UNSUPPORTED


def test_workspace_sizes(lib):
    ws = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LINEAR, 1, 1024, 2048, 2048, 4)
    assert ws >= 1024 * 2048 + 1024 * 64 * 4 and ws % 256 == 0
    wl = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD, 4, 1024, 2048, 2048, 4)
    assert wl >= 4 * 1024 * 2048
    with pytest.raises(loopq.LoopQError) as e:
        loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD, 65, 1, 32, 32, 4)
    assert e.value.status == loopq.LOOPQ_ERR_UNSUPPORTED


def _raw(lib, name, *args):
    return getattr(lib, name)(*args)


FAKE = 1 << 20  # a non-null, aligned address; never dereferenced because validation fails first


@pytest.mark.parametrize("K,n1,n2,bits,clip,want", [
    (33, 0, 0, 4, 1.0, loopq.LOOPQ_ERR_UNSUPPORTED),      # K % 32
    (256, 16, 8, 4, 1.0, loopq.LOOPQ_ERR_UNSUPPORTED),    # n1 * n2 != K
    (240, 16, 15, 4, 1.0, loopq.LOOPQ_ERR_UNSUPPORTED),   # n2 % 4 (K % 32 != 0 first: 240 ok)
    (256, 16, 16, 5, 1.0, loopq.LOOPQ_ERR_UNSUPPORTED),   # bits
    (256, 16, 16, 4, 0.0, loopq.LOOPQ_ERR_INVALID_ARG),   # clip <= 0
    (256, 16, 16, 4, float("nan"), loopq.LOOPQ_ERR_INVALID_ARG),
    (256, 16, 16, 4, float("inf"), loopq.LOOPQ_ERR_INVALID_ARG),
    (16384, 128, 128, 4, 1.0, loopq.LOOPQ_ERR_UNSUPPORTED),  # transform does not fit LDS
])
def test_quant_act_rejects_on_host(lib, K, n1, n2, bits, clip, want):
    p1 = FAKE if n1 else None
    p2 = FAKE if n2 else None
    st = _raw(lib, "loopq_quant_act", FAKE, loopq.LOOPQ_F32, 4, K, p1, n1, p2, n2, clip, bits,
              FAKE, FAKE, None, None)
    assert st == want


def test_quant_act_other_rejections(lib):
    # one factor without the other
    assert _raw(lib, "loopq_quant_act", FAKE, 0, 4, 256, FAKE, 16, None, 0, 1.0, 4, FAKE, FAKE,
                None, None) == loopq.LOOPQ_ERR_INVALID_ARG
    # bad dtype
    assert _raw(lib, "loopq_quant_act", FAKE, 7, 4, 256, None, 0, None, 0, 1.0, 4, FAKE, FAKE,
                None, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    # misaligned input (fp32 needs 16 bytes)
    assert _raw(lib, "loopq_quant_act", FAKE + 4, 0, 4, 256, None, 0, None, 0, 1.0, 4, FAKE, FAKE,
                None, None) == loopq.LOOPQ_ERR_ALIGNMENT
    # null outputs
    assert _raw(lib, "loopq_quant_act", FAKE, 0, 4, 256, None, 0, None, 0, 1.0, 4, None, FAKE,
                None, None) == loopq.LOOPQ_ERR_INVALID_ARG
    # M == 0 is an empty no-op (nothing is touched)
    assert _raw(lib, "loopq_quant_act", None, 0, 0, 256, None, 0, None, 0, 1.0, 4, None, None,
                None, None) == loopq.LOOPQ_OK
    # negative M
    assert _raw(lib, "loopq_quant_act", FAKE, 0, -1, 256, None, 0, None, 0, 1.0, 4, FAKE, FAKE,
                None, None) == loopq.LOOPQ_ERR_INVALID_ARG


def test_looped_forward_rejects_on_host(lib):
    clips = (ctypes.c_float * 2)(1.0, 0.5)
    bad = (ctypes.c_float * 2)(1.0, -0.5)
    args = lambda T, c, gw=32, sched=0, ws=1 << 30: (FAKE, 0, T, 4, 256, 128, None, 0, None, 0,
                                                      ctypes.cast(c, ctypes.c_void_p), 4, FAKE, FAKE,
                                                      gw, FAKE, sched, FAKE, ws, None)
    assert _raw(lib, "loopq_looped_forward", *args(0, clips)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert _raw(lib, "loopq_looped_forward", *args(65, clips)) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert _raw(lib, "loopq_looped_forward", *args(2, bad)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert _raw(lib, "loopq_looped_forward", *args(2, clips, gw=64)) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert _raw(lib, "loopq_looped_forward", *args(2, clips, sched=3)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert _raw(lib, "loopq_looped_forward", *args(2, clips, ws=16)) == loopq.LOOPQ_ERR_WORKSPACE


def test_pack_and_fold_reject_on_host(lib):
    assert _raw(lib, "loopq_pack_weights", FAKE, 48, 8, 32, FAKE, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert _raw(lib, "loopq_pack_weights", FAKE, 64, 8, 32, FAKE + 8, FAKE, None) == loopq.LOOPQ_ERR_ALIGNMENT
    assert _raw(lib, "loopq_pack_weights", None, 64, 8, 32, FAKE, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert _raw(lib, "loopq_fold_weights", FAKE, 256, 8, FAKE, 16, FAKE, 8, FAKE, FAKE, 1 << 30,
                None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert _raw(lib, "loopq_fold_weights", FAKE, 256, 8, FAKE, 16, FAKE, 16, FAKE, FAKE, 16,
                None) == loopq.LOOPQ_ERR_WORKSPACE


def test_looped_forward_ex_rejects_on_host(lib):
    T = 3
    VP = ctypes.c_void_p * 2
    wc, wsc = VP(FAKE, FAKE), VP(FAKE, FAKE)
    arr = lambda ct, vals: ctypes.cast((ct * len(vals))(*vals), ctypes.c_void_p)
    def call(sets, bits, clips=(1.0, 0.9, 0.8), nsets=2, codes=wc, ws=1 << 30):
        return _raw(lib, "loopq_looped_forward_ex", FAKE, 0, T, 4, 256, 128, nsets, None, 0, None, 0,
                    ctypes.cast(codes, ctypes.c_void_p), ctypes.cast(wsc, ctypes.c_void_p), 32,
                    arr(ctypes.c_int32, sets), arr(ctypes.c_int32, bits), arr(ctypes.c_float, clips),
                    FAKE, FAKE, ws, None)
    assert call([0, 1, 2], [4, 4, 4]) == loopq.LOOPQ_ERR_INVALID_ARG   # set index past nsets
    assert call([0, -1, 0], [4, 4, 4]) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call([0, 1, 1], [4, 6, 4]) == loopq.LOOPQ_ERR_UNSUPPORTED   # bit width
    assert call([0, 1, 1], [4, 8, 4], clips=(1.0, 0.0, 1.0)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call([0, 0, 0], [4, 4, 4], nsets=0) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call([0, 1, 1], [4, 8, 4], codes=VP(FAKE, None)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call([0, 1, 1], [4, 8, 4], ws=16) == loopq.LOOPQ_ERR_WORKSPACE
    # enough for both bit widths
    need = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD_EX, 4, 64, 2048, 512, 0)
    assert need >= max(loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD, 4, 64, 2048, 512, b) for b in (4, 8))


def test_hessian_workspace_and_host_rejections(lib):
    op = loopq.LOOPQ_OP_HESSIAN
    # room for two 128 x 128 fp32 pieces per work group (512 of them) whenever
    # the tiles on or above the diagonal are not a multiple of 512: K = 2048
    # has 136, K = 4096 has 528, K = 65536 has 131328
    for K in (32, 2048, 4096, 65536):
        assert loopq.loopq_workspace_bytes(op, 0, 16, K, 0, 0) == 512 * 2 * 128 * 128 * 4
    for K, want in ((48, loopq.LOOPQ_ERR_UNSUPPORTED), (65536 + 32, loopq.LOOPQ_ERR_UNSUPPORTED),
                    (0, loopq.LOOPQ_ERR_INVALID_ARG)):
        with pytest.raises(loopq.LoopQError) as e:
            loopq.loopq_workspace_bytes(op, 0, 16, K, 0, 0)
        assert e.value.status == want
    ws = 512 * 2 * 128 * 128 * 4
    call = lambda x, rows, K, H, w=FAKE, nb=ws: _raw(lib, "loopq_hessian_accumulate", x, rows, K, H, w, nb, None)
    assert call(FAKE, -1, 256, FAKE) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(FAKE, 8, 0, FAKE) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(FAKE, 8, 48, FAKE) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(FAKE, 8, 65536 + 32, FAKE) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(FAKE, (1 << 30) + 1, 256, FAKE) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(None, 8, 256, FAKE) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(FAKE, 8, 256, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(FAKE + 8, 8, 256, FAKE) == loopq.LOOPQ_ERR_ALIGNMENT   # xt needs 16 bytes
    assert call(FAKE, 8, 256, FAKE + 2) == loopq.LOOPQ_ERR_ALIGNMENT
    assert call(FAKE, 8, 2048, FAKE, nb=ws - 1) == loopq.LOOPQ_ERR_WORKSPACE
    assert call(FAKE, 8, 2048, FAKE, w=None) == loopq.LOOPQ_ERR_WORKSPACE
    assert call(FAKE, 8, 2048, FAKE, w=FAKE + 16) == loopq.LOOPQ_ERR_ALIGNMENT
    # no rows: nothing to add, nothing enqueued, whatever the pointers
    assert call(FAKE, 0, 2048, FAKE) == loopq.LOOPQ_OK
    assert call(None, 0, 2048, None, w=None) == loopq.LOOPQ_OK


def test_per_token_entries_reject_on_host(lib):
    qop, lop = loopq.LOOPQ_OP_QUANT_PER_TOKEN, loopq.LOOPQ_OP_LOOPED_FORWARD_PER_TOKEN
    assert loopq.loopq_workspace_bytes(qop, 0, 100, 2048, 0, 0) == 0  # the call needs none
    # the loop: the group path's activation buffers for T*M rows
    assert loopq.loopq_workspace_bytes(lop, 3, 100, 2048, 512, 4) == \
        loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LINEAR, 1, 300, 2048, 512, 4)
    for args, want in (((lop, 3, 100, 2048, 512, 5), loopq.LOOPQ_ERR_UNSUPPORTED),
                       ((lop, 65, 1, 2048, 512, 4), loopq.LOOPQ_ERR_UNSUPPORTED),
                       ((lop, 0, 1, 2048, 512, 4), loopq.LOOPQ_ERR_INVALID_ARG)):
        with pytest.raises(loopq.LoopQError) as e:
            loopq.loopq_workspace_bytes(*args)
        assert e.value.status == want
    q = lambda *a: _raw(lib, "loopq_quant_act_per_token", *a)
    # x, dtype, M, K, P1, n1, P2, n2, clip, bits, codes, scales, xt_out, ws, ws_bytes, stream
    assert q(FAKE, 0, 4, 48, None, 0, None, 0, 1.0, 4, FAKE, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 256, None, 0, None, 0, 0.0, 4, FAKE, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert q(FAKE, 0, 4, 256, None, 0, None, 0, 1.0, 6, FAKE, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 256, None, 0, None, 0, 1.0, 4, None, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert q(FAKE, 0, 4, 256, None, 0, None, 0, 1.0, 4, FAKE + 2, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_ALIGNMENT
    # a transform with no x~ output needs no workspace either: only the
    # factor checks run (n1 * n2 != K is rejected before any launch)
    assert q(FAKE, 0, 4, 256, FAKE, 16, FAKE, 8, 1.0, 4, FAKE, FAKE, None, None, 0, None) == \
        loopq.LOOPQ_ERR_UNSUPPORTED
    assert q(FAKE, 0, 4, 256, FAKE, 16, FAKE, 8, 1.0, 4, FAKE, FAKE, None, None, 0, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert q(FAKE, 0, 0, 256, None, 0, None, 0, 1.0, 4, None, None, None, None, 0, None) == loopq.LOOPQ_OK
    arr = lambda vals: ctypes.cast((ctypes.c_float * len(vals))(*vals), ctypes.c_void_p)
    lp = lambda T, clips, gw=32, ws=1 << 30, wc=FAKE: _raw(
        lib, "loopq_looped_forward_per_token", FAKE, 0, T, 4, 256, 128, None, 0, None, 0, arr(clips), 4, wc, FAKE,
        gw, FAKE, FAKE, ws, None)
    assert lp(2, [1.0, 0.9], gw=64) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert lp(2, [1.0, 0.9], ws=16) == loopq.LOOPQ_ERR_WORKSPACE
    assert lp(2, [1.0, 0.9], wc=None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert lp(2, [1.0, float("nan")]) == loopq.LOOPQ_ERR_INVALID_ARG
    assert lp(0, [1.0]) == loopq.LOOPQ_ERR_INVALID_ARG
    assert lp(65, [1.0] * 65) == loopq.LOOPQ_ERR_UNSUPPORTED


def test_recurrent_adapter_rejects_on_host(lib):
    op = loopq.LOOPQ_OP_RECURRENT_ADAPTER
    # x = cat(s, e) staging plus the linear's buffers for K = 2N
    assert loopq.loopq_workspace_bytes(op, 0, 16, 0, 5280, 8) == \
        16 * 10560 * 4 + loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LINEAR, 1, 16, 10560, 5280, 8)
    with pytest.raises(loopq.LoopQError) as e:
        loopq.loopq_workspace_bytes(op, 0, 16, 0, 72, 8)     # N % 16
    assert e.value.status == loopq.LOOPQ_ERR_UNSUPPORTED
    arr = lambda vals: ctypes.cast((ctypes.c_float * len(vals))(*vals), ctypes.c_void_p)
    def call(T=2, M=4, N=64, clips=(1.0, 0.9), gw=32, ws=1 << 30, e=FAKE, s0=FAKE, bits=4):
        return _raw(lib, "loopq_recurrent_adapter", s0, e, T, M, N, None, 0, None, 0, arr(list(clips)), bits, FAKE,
                    FAKE, gw, FAKE, FAKE, ws, None)
    assert call(N=72) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(T=0, clips=(1.0,)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(T=65, clips=(1.0,) * 65) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(clips=(1.0, -1.0)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(gw=64) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(bits=6) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert call(e=None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert call(e=FAKE + 8) == loopq.LOOPQ_ERR_ALIGNMENT
    assert call(s0=FAKE + 4) == loopq.LOOPQ_ERR_ALIGNMENT
    assert call(ws=16) == loopq.LOOPQ_ERR_WORKSPACE
    assert call(M=0, e=None, s0=None) == loopq.LOOPQ_OK


def test_export_act_codes_rejects_on_host(lib):
    x = lambda *a: _raw(lib, "loopq_export_act_codes", *a)
    op = loopq.LOOPQ_OP_LOOPED_FORWARD
    ws = loopq.loopq_workspace_bytes(op, 4, 64, 2048, 512, 4)
    # workspace, bytes, op, T, M, K, N, bits, schedule, codes, scales, stream
    assert x(FAKE, ws, 99, 4, 64, 2048, 512, 4, 0, FAKE, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert x(FAKE, ws, loopq.LOOPQ_OP_LINEAR, 2, 64, 2048, 512, 4, 0, FAKE, FAKE, None) == \
        loopq.LOOPQ_ERR_INVALID_ARG
    assert x(FAKE, ws, op, 4, 64, 2048, 512, 6, 0, FAKE, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert x(FAKE, ws, op, 4, 64, 2040, 512, 4, 0, FAKE, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert x(FAKE, ws, op, 4, 64, 2048, 512, 4, 3, FAKE, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert x(FAKE, ws - 1, op, 4, 64, 2048, 512, 4, 0, FAKE, FAKE, None) == loopq.LOOPQ_ERR_WORKSPACE
    assert x(FAKE + 16, ws, op, 4, 64, 2048, 512, 4, 0, FAKE, FAKE, None) == loopq.LOOPQ_ERR_ALIGNMENT
    assert x(FAKE, ws, op, 4, 64, 2048, 512, 4, 0, None, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert x(FAKE, ws, op, 4, 64, 2048, 512, 4, 0, FAKE, FAKE + 2, None) == loopq.LOOPQ_ERR_ALIGNMENT
    assert x(None, 0, op, 4, 0, 2048, 512, 4, 0, None, None, None) == loopq.LOOPQ_OK  # no rows
    w = lambda *a: _raw(lib, "loopq_export_weight_codes", *a)
    assert w(FAKE, 2040, 64, 32, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert w(FAKE, 2048, 64, 64, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert w(None, 2048, 64, 32, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert w(FAKE + 8, 2048, 64, 32, FAKE, None) == loopq.LOOPQ_ERR_ALIGNMENT


def test_noalloc_linear_rejects_on_host(lib):
    """Argument errors and a call larger than the fixed scratch return before
    any HIP call (this runs without a GPU)."""
    f = lambda *a: _raw(lib, "loopq_w4a4_linear_noalloc", *a)
    assert loopq.loopq_noalloc_scratch_bytes() == 64 << 20
    # x, dtype, M, K, N, P1, n1, P2, n2, clip, bits, w_codes, w_scales, group_w, y, stream
    assert f(FAKE, 0, 4, 48, 64, None, 0, None, 0, 1.0, 4, FAKE, FAKE, 32, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert f(FAKE, 0, 4, 256, 64, None, 0, None, 0, 0.0, 4, FAKE, FAKE, 32, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert f(FAKE, 0, 4, 256, 64, None, 0, None, 0, 1.0, 6, FAKE, FAKE, 32, FAKE, None) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert f(FAKE, 0, 4, 256, 64, None, 0, None, 0, 1.0, 4, None, FAKE, 32, FAKE, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert f(FAKE, 0, 4, 256, 64, None, 0, None, 0, 1.0, 4, FAKE + 8, FAKE, 32, FAKE, None) == \
        loopq.LOOPQ_ERR_ALIGNMENT
    assert f(None, 0, 0, 256, 64, None, 0, None, 0, 1.0, 4, None, None, 32, None, None) == loopq.LOOPQ_OK  # no rows
    # 32768 rows at K = N = 2048 need more than 64 MiB of scratch
    need = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LINEAR, 1, 32768, 2048, 2048, 4)
    assert need > 64 << 20
    assert f(FAKE, 0, 32768, 2048, 2048, None, 0, None, 0, 1.0, 4, FAKE, FAKE, 32, FAKE, None) == \
        loopq.LOOPQ_ERR_WORKSPACE


def test_cta_entries_reject_on_host(lib):
    """Argument errors of the CTA calls return before any HIP call."""
    f = lambda *a: _raw(lib, "loopq_cta_apply", *a)
    # h, dtype, M, K, U, V, rank, a, b, eta, out, stream
    ok = (FAKE, 1, 4, 256, FAKE, FAKE, 8, FAKE, FAKE, 0.5, FAKE + (1 << 20), None)

    def vary(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert vary(1, 2) == loopq.LOOPQ_ERR_INVALID_ARG           # dtype
    assert vary(3, 250) == loopq.LOOPQ_ERR_UNSUPPORTED          # K % 32
    assert vary(6, 0) == loopq.LOOPQ_ERR_INVALID_ARG            # rank
    assert vary(6, 17) == loopq.LOOPQ_ERR_UNSUPPORTED           # rank above 16
    assert vary(9, float("nan")) == loopq.LOOPQ_ERR_INVALID_ARG
    assert vary(4, None) == loopq.LOOPQ_ERR_INVALID_ARG
    assert vary(0, FAKE + 8) == loopq.LOOPQ_ERR_ALIGNMENT
    assert vary(7, FAKE + 2) == loopq.LOOPQ_ERR_ALIGNMENT
    assert vary(10, FAKE + 16) == loopq.LOOPQ_ERR_INVALID_ARG   # out overlaps h, not in place
    assert vary(2, 0) == loopq.LOOPQ_OK                         # no rows
    g = lambda *a: _raw(lib, "loopq_looped_forward_cta", *a)
    op = loopq.LOOPQ_OP_LOOPED_FORWARD_CTA
    ws = loopq.loopq_workspace_bytes(op, 4, 64, 2048, 512, 4)
    base = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD, 4, 64, 2048, 512, 4)
    assert ws >= base + 4 * 64 * 2048 * 4
    clips = (ctypes.c_float * 4)(1.0, 1.0, 1.0, 1.0)
    etas = (ctypes.c_float * 3)(0.1, 0.2, 0.3)
    bad_etas = (ctypes.c_float * 3)(0.1, float("inf"), 0.3)
    # x, dtype, T, M, K, N, P1, n1, P2, n2, clips, bits, w_codes, w_scales, group_w, y, schedule,
    # U, V, rank, a_sets, b_sets, etas, workspace, bytes, stream
    base_args = [FAKE, 1, 4, 64, 2048, 512, None, 0, None, 0, ctypes.cast(clips, ctypes.c_void_p), 4, FAKE, FAKE,
                 32, FAKE, 0, FAKE, FAKE, 8, FAKE, FAKE, ctypes.cast(etas, ctypes.c_void_p), FAKE, ws, None]

    def gv(**kw):
        a = list(base_args)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return g(*a)
    assert gv(i19=0) == loopq.LOOPQ_ERR_INVALID_ARG                 # rank
    assert gv(i19=17) == loopq.LOOPQ_ERR_UNSUPPORTED
    assert gv(i17=None) == loopq.LOOPQ_ERR_INVALID_ARG              # U
    assert gv(i22=ctypes.cast(bad_etas, ctypes.c_void_p)) == loopq.LOOPQ_ERR_INVALID_ARG
    assert gv(i20=FAKE + 2) == loopq.LOOPQ_ERR_ALIGNMENT
    assert gv(i24=ws - 1) == loopq.LOOPQ_ERR_WORKSPACE
    assert gv(i23=FAKE + 16) == loopq.LOOPQ_ERR_ALIGNMENT
    assert gv(i4=2040) == loopq.LOOPQ_ERR_UNSUPPORTED              # K % 32
    assert gv(i3=0, i0=None, i23=None, i24=0) == loopq.LOOPQ_OK     # no rows


def test_forward_hessian_rejects_on_host(lib):
    f = lambda *a: _raw(lib, "loopq_looped_forward_hessian", *a)
    op = loopq.LOOPQ_OP_LOOPED_FORWARD_HESSIAN
    ws = loopq.loopq_workspace_bytes(op, 4, 64, 2048, 512, 4)
    base = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_LOOPED_FORWARD, 4, 64, 2048, 512, 4)
    hw = loopq.loopq_workspace_bytes(loopq.LOOPQ_OP_HESSIAN, 0, 256, 2048, 0, 0)
    assert ws >= base + 4 * 64 * 2048 * 4 + hw
    clips = (ctypes.c_float * 4)(1.0, 1.0, 1.0, 1.0)
    c = ctypes.cast(clips, ctypes.c_void_p)
    # x, dtype, T, M, K, N, P1, n1, P2, n2, clips, bits, w_codes, w_scales, group_w, y, schedule, H, ws, bytes, stream
    args = [FAKE, 1, 4, 64, 2048, 512, None, 0, None, 0, c, 4, FAKE, FAKE, 32, FAKE, 0, FAKE, FAKE, ws, None]

    def v(i, x):
        a = list(args)
        a[i] = x
        return f(*a)
    assert v(17, None) == loopq.LOOPQ_ERR_INVALID_ARG        # H
    assert v(17, FAKE + 2) == loopq.LOOPQ_ERR_ALIGNMENT
    assert v(19, ws - 1) == loopq.LOOPQ_ERR_WORKSPACE
    assert v(18, FAKE + 16) == loopq.LOOPQ_ERR_ALIGNMENT
    assert v(4, 2040) == loopq.LOOPQ_ERR_UNSUPPORTED          # K % 32
    assert v(16, 7) == loopq.LOOPQ_ERR_INVALID_ARG            # schedule
    with pytest.raises(loopq.LoopQError):
        loopq.loopq_workspace_bytes(op, 4, 64, 65568, 512, 4)  # K above the Hessian's limit
    a = list(args)
    a[3], a[0], a[17], a[18], a[19] = 0, None, None, None, 0
    assert f(*a) == loopq.LOOPQ_OK                             # no rows
