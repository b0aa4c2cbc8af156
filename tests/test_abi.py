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
    for path in (attn.LIB_PATH, attn.DEBUG_LIB_PATH):
        if not os.path.exists(path):
            assert path == attn.DEBUG_LIB_PATH, f"{path} not built"
            continue
        lib = ctypes.CDLL(path)
        for n in names:
            assert hasattr(lib, n), f"{n} declared in attn.h but not exported by {os.path.basename(path)}"
    assert set(names) == set(attn.EXPORTS)


def test_release_library_has_no_address_checks():
    """attn_debug_take belongs to the debug build: the release library says so
    without touching a device or the output."""
    out = (ctypes.c_ulonglong * 2)(7, 9)
    assert attn.lib().attn_debug_take(out) == attn.ATTN_ERR_UNSUPPORTED
    assert b"libattn_debug.so" in attn.lib().attn_last_error()
    assert (out[0], out[1]) == (7, 9)
    with pytest.raises(attn.AttnError):
        attn.debug_take()
    assert attn.lib().attn_debug_selftest(None) == attn.ATTN_ERR_UNSUPPORTED


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
    # partial dK and dV ([4][B, Tkv, Hkv, D] each) are summed afterwards; last,
    # 256 bytes of work counters for the dK/dV pass.
    queue = 256
    assert need == 6 * stat + 2 * 4 * (2 * 128 * 2 * 128) * 4 + queue
    assert L.attn_bwd_workspace_size(ctypes.byref(P(Hkv=8))) == 6 * stat + queue  # no group: no split
    big = P(B=4, Tq=8192, Tkv=8192, Hq=32, Hkv=8)  # 4 * 8 * 64 = 2048 workgroups: no split
    assert L.attn_bwd_workspace_size(ctypes.byref(big)) == 6 * (4 * 32 * 8192 * 4) + queue
    assert L.attn_bwd(ctypes.byref(p), *args, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd(ctypes.byref(p), *args, FAKE, need - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd(ctypes.byref(p), None, *args[1:], FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, need - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_preprocess(ctypes.byref(p), FAKE, None, FAKE, FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_dkdv(ctypes.byref(p), *([FAKE] * 7), None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_dkdv(ctypes.byref(p), *([FAKE] * 6), None, FAKE, need, None) == attn.ATTN_ERR_INVALID
    assert L.attn_bwd_dq(ctypes.byref(p), *([FAKE] * 6), FAKE, need - 4, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_dq(ctypes.byref(p), MISALIGNED, *([FAKE] * 5), FAKE, need, None) == attn.ATTN_ERR_INVALID
    # dQ with the preprocess outputs: q, k, v, o, lse, dout, dq, then the workspace.
    assert L.attn_bwd_dq_and_preprocess(ctypes.byref(p), *([FAKE] * 7), FAKE, need - 1, None) == \
        attn.ATTN_ERR_WORKSPACE
    assert L.attn_bwd_dq_and_preprocess(ctypes.byref(p), *([FAKE] * 3), None, *([FAKE] * 3), FAKE, need, None) == \
        attn.ATTN_ERR_INVALID
    assert L.attn_bwd_dq_and_preprocess(ctypes.byref(bad), *([FAKE] * 7), FAKE, need, None) == attn.ATTN_ERR_INVALID
    d = P(Tq=16, Tkv=16384, Hq=32, Hkv=8)
    s = L.attn_decode_num_splits(ctypes.byref(d))
    assert s >= 2
    wneed = L.attn_decode_workspace_size(ctypes.byref(d), 0)
    assert wneed == L.attn_decode_workspace_size(ctypes.byref(d), s) > 0
    assert L.attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, wneed - 1, None) == attn.ATTN_ERR_WORKSPACE
    assert L.attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, -1, FAKE, wneed, None) == attn.ATTN_ERR_INVALID
    dc = P(Tq=16, Tkv=16384, Hq=32, Hkv=8, causal=False, dtype=attn.ATTN_FP32)
    assert L.attn_decode(ctypes.byref(dc), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, wneed, None) == attn.ATTN_ERR_UNSUPPORTED
    # The decode kernels count key tiles of all segments in 32 bits: 2^14
    # segments (2^20 queries in 64-row blocks) of 2^17 key tiles each are
    # refused before any launch.
    dbig = P(B=1, Tq=1 << 20, Tkv=1 << 23, Hq=1, Hkv=1)
    assert L.attn_decode(ctypes.byref(dbig), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 1 << 40, None) == \
        attn.ATTN_ERR_UNSUPPORTED
    assert b"2^31" in L.attn_last_error()


def test_status_strings():
    L = attn.lib()
    for s in range(5):
        assert L.attn_status_string(s)
    assert L.attn_status_string(99) == b"unknown status"


class _Launched(Exception):
    """Raised by the stand-in of a compute entry point: validation let the call through."""


class _NoLaunchLib:
    """The real library for host-only queries; every entry point that would
    launch a kernel raises instead."""

    COMPUTE = {"attn_fwd", "attn_bwd", "attn_bwd_preprocess", "attn_bwd_dkdv", "attn_bwd_dq", "attn_decode"}

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in self.COMPUTE:
            def launch(*args):
                raise _Launched(name)
            return launch
        return getattr(self._real, name)


@pytest.fixture
def host_binding(monkeypatch):
    """The binding with host tensors standing in for device tensors and no launches."""
    import torch
    monkeypatch.setattr(attn, "_on_device", lambda t: True)
    monkeypatch.setattr(attn, "_lib", _NoLaunchLib(attn.lib()))
    monkeypatch.setattr(attn, "_stream", lambda: None)
    return torch


def _bwd_problem(torch, dtype=None):
    dtype = dtype or torch.bfloat16
    B, T, Hq, Hkv, D = 2, 64, 4, 2, 64
    q = torch.zeros(B, T, Hq, D, dtype=dtype)
    k = torch.zeros(B, T, Hkv, D, dtype=dtype)
    lse = torch.zeros(B, Hq, T, dtype=torch.float32)
    return q, k, lse


def test_binding_lets_well_formed_calls_through(host_binding):
    torch = host_binding
    q, k, lse = _bwd_problem(torch)
    v, o, do = torch.zeros_like(k), torch.zeros_like(q), torch.zeros_like(q)
    for call in (lambda: attn.fwd(q, k, v),
                 lambda: attn.bwd(q, k, v, o, lse, do),
                 lambda: attn.bwd_dq(q, k, v, lse, do, attn.bwd_workspace(q, k), torch.zeros_like(q)),
                 lambda: attn.bwd_dkdv(q, k, v, lse, do, attn.bwd_workspace(q, k), torch.zeros_like(k),
                                       torch.zeros_like(k)),
                 lambda: attn.bwd_preprocess(o, lse, do, attn.bwd_workspace(q, k), q, k),
                 lambda: attn.decode(q[:, :4].contiguous(), k, v)):
        with pytest.raises(_Launched):
            call()


def test_binding_rejects_every_malformed_tensor_before_any_launch(host_binding):
    torch = host_binding
    q, k, lse = _bwd_problem(torch)
    v, o, do = torch.zeros_like(k), torch.zeros_like(q), torch.zeros_like(q)
    ws = attn.bwd_workspace(q, k)
    bad_lse = [lse.double(), lse[:, :, :-1], lse.transpose(1, 2).contiguous().transpose(1, 2), lse.to(torch.bfloat16)]
    bad_q_like = [q.float(), q[:, :-1], q.transpose(1, 2), torch.zeros(2, 64, 4, 32, dtype=torch.bfloat16)]
    bad_k_like = [k.float(), k[:, :-1], k.transpose(1, 2), torch.zeros_like(q)]
    cases = []
    for bl in bad_lse:
        cases += [lambda bl=bl: attn.fwd(q, k, v, lse=bl),
                  lambda bl=bl: attn.bwd(q, k, v, o, bl, do),
                  lambda bl=bl: attn.bwd_preprocess(o, bl, do, ws, q, k),
                  lambda bl=bl: attn.bwd_dkdv(q, k, v, bl, do, ws, torch.zeros_like(k), torch.zeros_like(k)),
                  lambda bl=bl: attn.bwd_dq(q, k, v, bl, do, ws, torch.zeros_like(q)),
                  lambda bl=bl: attn.bwd_dq_and_preprocess(q, k, v, o, bl, do, ws, torch.zeros_like(q))]
    for bq in bad_q_like:
        cases += [lambda bq=bq: attn.fwd(q, k, v, out=bq),
                  lambda bq=bq: attn.bwd(q, k, v, bq, lse, do),
                  lambda bq=bq: attn.bwd(q, k, v, o, lse, bq),
                  lambda bq=bq: attn.bwd_preprocess(bq, lse, do, ws, q, k),
                  lambda bq=bq: attn.bwd_preprocess(o, lse, bq, ws, q, k),
                  lambda bq=bq: attn.bwd_dq(q, k, v, lse, bq, ws, torch.zeros_like(q)),
                  lambda bq=bq: attn.bwd_dq(q, k, v, lse, do, ws, bq),
                  lambda bq=bq: attn.bwd_dq_and_preprocess(q, k, v, bq, lse, do, ws, torch.zeros_like(q)),
                  lambda bq=bq: attn.bwd_dq_and_preprocess(q, k, v, o, lse, bq, ws, torch.zeros_like(q)),
                  lambda bq=bq: attn.bwd_dq_and_preprocess(q, k, v, o, lse, do, ws, bq)]
    for bk in bad_k_like:
        cases += [lambda bk=bk: attn.fwd(q, k, bk),
                  lambda bk=bk: attn.bwd(q, k, bk, o, lse, do),
                  lambda bk=bk: attn.bwd_dkdv(q, k, bk, lse, do, ws, torch.zeros_like(k), torch.zeros_like(k)),
                  lambda bk=bk: attn.bwd_dkdv(q, k, v, lse, do, ws, bk, torch.zeros_like(k)),
                  lambda bk=bk: attn.bwd_dkdv(q, k, v, lse, do, ws, torch.zeros_like(k), bk),
                  lambda bk=bk: attn.bwd_dq(q, k, bk, lse, do, ws, torch.zeros_like(q)),
                  lambda bk=bk: attn.bwd_dq_and_preprocess(q, k, bk, o, lse, do, ws, torch.zeros_like(q)),
                  lambda bk=bk: attn.decode(q, k, bk)]
    small_ws = ws[:-1]
    cases += [lambda: attn.bwd(q, k, v, o, lse, do, workspace=small_ws),
              lambda: attn.bwd_preprocess(o, lse, do, small_ws, q, k),
              lambda: attn.bwd_dkdv(q, k, v, lse, do, small_ws, torch.zeros_like(k), torch.zeros_like(k)),
              lambda: attn.bwd_dq(q, k, v, lse, do, small_ws, torch.zeros_like(q)),
              lambda: attn.bwd_dq_and_preprocess(q, k, v, o, lse, do, small_ws, torch.zeros_like(q)),
              lambda: attn.bwd_dq(q, k, v, lse, do, ws[::2], torch.zeros_like(q)),
              lambda: attn.bwd_dq(q, k, v, lse, do, "not a tensor", torch.zeros_like(q)),
              lambda: attn.fwd(q, k, v, kv_lens=torch.zeros(2, dtype=torch.int64)),
              lambda: attn.fwd(q, k, v, kv_lens=torch.zeros(3, dtype=torch.int32)),
              lambda: attn.fwd(q, k, v, kv_lens=torch.zeros(2, 1, dtype=torch.int32))]
    for i, call in enumerate(cases):
        with pytest.raises(ValueError):
            call()


def test_binding_counts_workspace_bytes_not_elements(host_binding):
    torch = host_binding
    q, k, lse = _bwd_problem(torch)
    need = attn.lib().attn_bwd_workspace_size(ctypes.byref(attn.make_params(2, 64, 64, 4, 2, 64)))
    ws32 = torch.zeros((need + 3) // 4, dtype=torch.float32)  # enough bytes in fewer elements
    with pytest.raises(_Launched):
        attn.bwd_dq(q, k, torch.zeros_like(k), lse, torch.zeros_like(q), ws32, torch.zeros_like(q))


def test_workspace_errors_report_sizes_above_2_gib():
    """Workspace sizes print as size_t: a 12 GiB backward workspace and a
    decode workspace past 2^32 bytes are quoted exactly."""
    L = attn.lib()
    p = P(B=1024, Tq=65536, Tkv=65536, Hq=8, Hkv=8)
    need = L.attn_bwd_workspace_size(ctypes.byref(p))
    assert need == 6 * 1024 * 8 * 65536 * 4 + 256 > 2**33
    assert L.attn_bwd(ctypes.byref(p), *([FAKE] * 9), FAKE, 1, None) == attn.ATTN_ERR_WORKSPACE
    assert f"{need} bytes needed, 1 given".encode() in L.attn_last_error()
    d = P(B=32768, Tq=1, Tkv=1024, Hq=32, Hkv=8)  # 262144 segments, the most the counters take
    wneed = L.attn_decode_workspace_size(ctypes.byref(d), 0)
    assert wneed > 2**32
    assert L.attn_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, wneed - 16, None) == \
        attn.ATTN_ERR_WORKSPACE
    assert f"{wneed} bytes needed, {wneed - 16} given".encode() in L.attn_last_error()


def test_noalloc_decode_rejects_oversized_calls_before_touching_a_device():
    """Calls whose workspace would exceed the static scratch are refused on the
    host, and so are malformed ones, with no HIP call made (none is possible here)."""
    L = attn.lib()
    d = P(B=8, Tq=256, Tkv=65536, Hq=32, Hkv=32)  # 8 * 32 * 4 row blocks = 1024 segments
    need = L.attn_decode_workspace_size(ctypes.byref(d), 0)
    assert need > (32 << 20)
    assert L.attn_decode_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, None) == attn.ATTN_ERR_WORKSPACE
    assert f"needs {need} bytes of scratch".encode() in L.attn_last_error()
    assert f"holds {32 << 20}".encode() in L.attn_last_error()
    ok = P(Tq=16, Tkv=16384, Hq=32, Hkv=8)
    assert L.attn_decode_noalloc(ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, None, 2**30, None) == \
        attn.ATTN_ERR_WORKSPACE
    assert L.attn_decode_noalloc(ctypes.byref(ok), None, FAKE, FAKE, FAKE, None, 0, None) == attn.ATTN_ERR_INVALID
    assert L.attn_decode_noalloc(ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, None, -1, None) == attn.ATTN_ERR_INVALID
    assert L.attn_decode_noalloc(ctypes.byref(P(causal=True)), FAKE, FAKE, FAKE, FAKE, None, 0, None) == \
        attn.ATTN_ERR_INVALID

