"""The C ABI on a host without a GPU: library load, exports, validation (no device calls)."""

import ctypes
import os
import re

import pytest

from forward_backward_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(attn.LIB_PATH), reason="libattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert "attn_fwd" in names and "attn_bwd" in names and "attn_decode" in names
    lib = ctypes.CDLL(attn.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in attn.h but not exported"
    assert set(names) == set(attn.EXPORTS)


def P(**kw):
    base = dict(B=2, Tq=128, Tkv=128, Hq=8, Hkv=2, D=128, dtype=attn.ATTN_BF16, scale=0.125, causal=False)
    base.update(kw)
    return attn.make_params(**base)


def validate(p, op=attn.OP_FWD):
    return attn.lib().attn_validate(ctypes.byref(p), op)


@pytest.mark.parametrize("kw,op,status", [
    ({}, attn.OP_FWD, attn.ATTN_OK),
    ({}, attn.OP_BWD, attn.ATTN_OK),
    ({"Tq": 16, "Tkv": 4096}, attn.OP_DECODE, attn.ATTN_OK),
    ({"B": 0}, attn.OP_FWD, attn.ATTN_OK),
    ({"Tkv": 0}, attn.OP_FWD, attn.ATTN_OK),
    ({"B": -1}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"Hq": 0}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"Hq": 6, "Hkv": 4}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"causal": True, "Tq": 64}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"causal": True}, attn.OP_DECODE, attn.ATTN_ERR_INVALID),
    ({"scale": 0.0}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"scale": -0.5}, attn.OP_BWD, attn.ATTN_ERR_INVALID),
    ({"scale": float("nan")}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"scale": float("inf")}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"D": 96}, attn.OP_FWD, attn.ATTN_ERR_UNSUPPORTED),
    ({"D": 32}, attn.OP_FWD, attn.ATTN_OK),
    ({"D": 32, "Tq": 16, "Tkv": 4096}, attn.OP_DECODE, attn.ATTN_OK),
    ({"D": 32, "dtype": attn.ATTN_FP32}, attn.OP_BWD, attn.ATTN_OK),
    ({"D": 256}, attn.OP_BWD, attn.ATTN_OK),
    ({"D": 256, "Tq": 16, "Tkv": 4096}, attn.OP_DECODE, attn.ATTN_OK),
    ({"D": 256, "dtype": attn.ATTN_FP32}, attn.OP_FWD, attn.ATTN_ERR_UNSUPPORTED),
    ({"D": 512}, attn.OP_FWD, attn.ATTN_ERR_UNSUPPORTED),
    ({"dtype": 7}, attn.OP_FWD, attn.ATTN_ERR_INVALID),
    ({"dtype": attn.ATTN_FP32}, attn.OP_DECODE, attn.ATTN_ERR_UNSUPPORTED),
    ({"dtype": attn.ATTN_FP32}, attn.OP_BWD, attn.ATTN_OK),
    ({"window": (16, 0)}, attn.OP_FWD, attn.ATTN_OK),
    ({"window": (-1, 3)}, attn.OP_BWD, attn.ATTN_OK),
    ({"window": (16, 0), "Tq": 64}, attn.OP_FWD, attn.ATTN_ERR_INVALID),      # windows need Tq == Tkv
    ({"window": (-1, -1), "Tq": 64}, attn.OP_FWD, attn.ATTN_OK),              # no window
    ({"window": (128, 500), "Tq": 64}, attn.OP_FWD, attn.ATTN_OK),            # reaches past every key
    ({"window": (8, -1), "Tq": 16, "Tkv": 4096}, attn.OP_DECODE, attn.ATTN_ERR_INVALID),
    ({"window": (8, 8)}, attn.OP_DECODE, attn.ATTN_ERR_INVALID),
])
def test_validate(kw, op, status):
    assert validate(P(**kw), op) == status


def test_validate_rejects_null_params_and_unknown_op():
    L = attn.lib()
    assert L.attn_validate(None, attn.OP_FWD) == attn.ATTN_ERR_INVALID
    assert L.attn_validate(ctypes.byref(P()), 9) == attn.ATTN_ERR_INVALID
    assert b"op" in L.attn_last_error()


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every case fails validation first
MISALIGNED = ctypes.c_void_p(0x1004)


def test_entry_points_reject_bad_arguments_before_any_launch():
    L = attn.lib()
    p = P()
    assert L.attn_fwd(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, None) == attn.ATTN_ERR_INVALID
    assert L.attn_fwd(ctypes.byref(p), MISALIGNED, FAKE, FAKE, FAKE, FAKE, None) == attn.ATTN_ERR_INVALID
    assert b"aligned" in L.attn_last_error()
    bad = P(Hq=5, Hkv=2)
    assert L.attn_fwd(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None) == attn.ATTN_ERR_INVALID
    args = [FAKE] * 9
    need = L.attn_bwd_workspace_size(ctypes.byref(p))
    # D and LSE * log2(e) (fp32 each) and 16 bytes of bf16 row terms per query row ...
    stat = 2 * 8 * 128 * 4
    # ... plus, since 2 batches x 2 KV heads x one 128-key tile leave the chip
    # idle, the 4 query heads of a group split over 4 workgroups whose fp32
    # partial dK and dV ([4][B, Tkv, Hkv, D] each) are summed afterwards.
    assert need == 6 * stat + 2 * 4 * (2 * 128 * 2 * 128) * 4
    assert L.attn_bwd_workspace_size(ctypes.byref(P(Hkv=8))) == 6 * stat  # no group: no split
    big = P(B=4, Tq=8192, Tkv=8192, Hq=32, Hkv=8)  # 4 * 8 * 64 = 2048 workgroups: no split
    assert L.attn_bwd_workspace_size(ctypes.byref(big)) == 6 * (4 * 32 * 8192 * 4)
    assert L.attn_bwd(ctypes.byref(p), *args, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd(ctypes.byref(p), *args, FAKE, need - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd(ctypes.byref(p), None, *args[1:], FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, need - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, None, FAKE, FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_dkdv(ctypes.byref(p), *([FAKE] * 7), None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_dkdv(ctypes.byref(p), *([FAKE] * 6), None, FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_dq(ctypes.byref(p), *([FAKE] * 6), FAKE, need - 4, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_dq(ctypes.byref(p), MISALIGNED, *([FAKE] * 5), FAKE, need, None) == attn.ATTN_ERR_INVALID
    d = P(Tq=16, Tkv=16384, Hq=32, Hkv=8)
    s = L.attn_decode_num_splits(ctypes.byref(d))
    assert s >= 2
    wneed = L.attn_decode_workspace_size(ctypes.byref(d), 0)
    assert wneed == L.attn_decode_workspace_size(ctypes.byref(d), s) > 0
    assert L.attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, wneed - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, -1, FAKE, wneed, None) == attn.ATTN_ERR_INVALID
    dc = P(Tq=16, Tkv=16384, Hq=32, Hkv=8, causal=False, dtype=attn.ATTN_FP32)
    assert L.attn_decode(ctypes.byref(dc), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, wneed, None) == attn.ATTN_ERR_UNSUPPORTED


def test_status_strings():
    L = attn.lib()
    for s in range(5):
        assert L.attn_status_string(s)
    assert L.attn_status_string(99) == b"unknown status"
