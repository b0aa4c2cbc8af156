"""The address-checking build (libattn_debug.so) on edge cases (needs an MI355X).

Every global load and global->LDS copy of its kernels checks the bytes it
reads against the buffers of the call; the cases below (ragged lengths, KV
lengths of 0, 1 and outside [0, Tkv], windows, head splits, every head_dim,
fp32, decode with its static scratch) must read nothing outside them, and
the checked build must give the release build's outputs bit for bit (the
checks change no arithmetic)."""

import contextlib
import ctypes

import pytest

from forward_backward_amd.inputs import Case
from helpers import device_inputs
from test_gpu_bwd import run_fwd_bwd

pytestmark = pytest.mark.gpu

FWD_BWD = [
    Case("dbg_d128_gqa_kvlen_out_of_range", 3, 200, 300, 8, 2, 128, kv_lens=(-3, 350, 299), workload_id=700),
    Case("dbg_d128_causal_T333", 2, 333, 333, 4, 2, 128, causal=True, workload_id=701),
    Case("dbg_d128_causal_window", 2, 700, 700, 4, 4, 128, causal=True, window=(100, 0), workload_id=702),
    Case("dbg_d128_two_sided_window", 1, 600, 600, 2, 2, 128, window=(50, 70), workload_id=703),
    Case("dbg_gqa32_head_split_T200", 1, 200, 200, 32, 1, 128, workload_id=704),
    Case("dbg_b16_d128_T64", 16, 64, 64, 4, 2, 128, workload_id=705),
    Case("dbg_d64_causal_kvlen", 2, 333, 333, 4, 4, 64, causal=True, kv_lens=(383, -1), workload_id=706),
    Case("dbg_d32_ragged", 2, 300, 260, 4, 2, 32, kv_lens=(260, 7), workload_id=707),
    Case("dbg_d256_kvlen", 1, 130, 130, 16, 1, 256, kv_lens=(77,), workload_id=708),
    Case("dbg_fp32_d64_kvlen_out_of_range", 2, 70, 90, 2, 1, 64, "fp32", kv_lens=(-7, 1000), workload_id=709),
    Case("dbg_fp32_d128_causal", 1, 150, 150, 2, 2, 128, "fp32", causal=True, workload_id=710),
]

DECODE = [
    Case("dbg_dec_q16_g4", 2, 16, 3000, 8, 2, 128, kv_lens=(1, 2999), workload_id=711, decode=True),
    Case("dbg_dec_d64_kv0", 2, 5, 2048, 16, 2, 64, kv_lens=(0, 2048), workload_id=712, decode=True),
    Case("dbg_dec_b70", 70, 1, 300, 2, 1, 64, kv_len_range=(0, 300), workload_id=713, decode=True),
    Case("dbg_dec_kvlen_out_of_range", 3, 4, 700, 8, 2, 128, kv_lens=(-5, 750, 1), workload_id=714, decode=True),
    Case("dbg_dec_d256", 1, 2, 900, 4, 1, 256, workload_id=715, decode=True),
]


@pytest.fixture(scope="module")
def debug_lib():
    from forward_backward_amd import attn
    return attn.load_library(attn.DEBUG_LIB_PATH)


@contextlib.contextmanager
def using(handle):
    """Route the binding's calls through `handle` for the duration."""
    from forward_backward_amd import attn
    saved = attn.lib()
    attn._lib = handle
    try:
        yield
    finally:
        attn._lib = saved


def same_bits(name, a, b):
    import torch
    if a is None or b is None:
        assert a is None and b is None, name
        return
    iview = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(a.view(iview), b.view(iview)), f"{name}: the checked build differs"


def checked(debug_lib, fn):
    """fn() through the checked build; fails on any read outside the buffers."""
    import torch
    from forward_backward_amd import attn
    with using(debug_lib):
        attn.debug_take(debug_lib)  # counts of earlier calls
        out = fn()
        torch.cuda.synchronize()
        count, first = attn.debug_take(debug_lib)
    assert count == 0, f"{count} lane reads outside the call's buffers, the first at {first:#x}"
    return out


def test_the_checks_count_accesses_outside_the_ranges(debug_lib):
    """Positive control: the self-test wave checks 64 addresses of which 32
    lie past its registered range (it reads none of them)."""
    import torch
    from forward_backward_amd import attn
    attn.debug_take(debug_lib)
    assert debug_lib.attn_debug_selftest(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == attn.ATTN_OK
    count, first = attn.debug_take(debug_lib)
    base = 1 << 40
    assert count == 32 and base + 512 <= first < base + 1024, (count, hex(first))
    assert attn.debug_take(debug_lib) == (0, 0)


@pytest.mark.parametrize("case", FWD_BWD, ids=lambda c: c.name)
def test_fwd_bwd_reads_stay_inside_the_buffers(case, debug_lib):
    import torch
    host, dev, _ = device_inputs(case)
    print(f"[address checks] {case.name}", flush=True)
    ref = run_fwd_bwd(case, dev)
    torch.cuda.synchronize()
    got = checked(debug_lib, lambda: run_fwd_bwd(case, dev))
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        same_bits(name, a, b)


@pytest.mark.parametrize("case", DECODE, ids=lambda c: c.name)
def test_decode_reads_stay_inside_the_buffers(case, debug_lib):
    import torch
    from forward_backward_amd import attn
    host, dev, _ = device_inputs(case, with_do=False)
    print(f"[address checks] {case.name}", flush=True)

    def run():
        return attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale)

    def run_noalloc():
        return attn.decode_noalloc(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale)

    ref = run()
    torch.cuda.synchronize()
    for fn in (run, run_noalloc):
        got = checked(debug_lib, fn)
        for name, a, b in zip(("o", "lse"), got, ref):
            same_bits(name, a, b)


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_debug_calls_refuse_graph_capture(debug_lib):
    """The checked build writes its address tables synchronously before a
    launch, which a captured graph could not replay: capture is refused
    with ATTN_ERR_UNSUPPORTED (and nothing is launched)."""
    import torch
    from forward_backward_amd import attn
    case = DECODE[0]
    host, dev, _ = device_inputs(case, with_do=False)
    ws = attn.decode_workspace(dev["q"], dev["k"])
    g = torch.cuda.CUDAGraph()
    with using(debug_lib):
        with pytest.raises(attn.AttnError) as err:
            with torch.cuda.graph(g):
                attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
    assert err.value.status == attn.ATTN_ERR_UNSUPPORTED
