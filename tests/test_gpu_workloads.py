"""Whole-tensor parity of the five workloads against the float64 oracle (needs an MI355X).

Every element of O, LSE, dQ, dK and dV is compared: the fp32 correctness case
(B1 H2 T128 d64), the bf16 head_dim-64 grid (B4 H8, six lengths, causal and
not), the headline shape (B4 H8 d128 T8192, causal and not), the KV-length
case (B4 H8 d128 T4096, lengths 1, 777, 2500, 4096) and the GQA decode case
(B4, 32 query heads over 8 KV heads, 16 queries over a 16384-key cache). The
metric is max|a - b| / max|b| per tensor ("GPU and CPU performance", section
"Methodology"), bounded by 1e-2 for bf16 and 1e-4 for fp32; LSE by 1e-4 on
finite entries with equal -inf positions.

The oracle runs per (batch, head) in a thread pool (tests/helpers.py); the
headline cases take about half a minute of host time each and are marked slow.
"""

import numpy as np
import pytest

from forward_backward_amd.inputs import Case, workload_cases
from helpers import compare_all, device_inputs, oracle_full, to_host64

pytestmark = pytest.mark.gpu


def run_fwd_bwd(case, dev):
    from forward_backward_amd import attn
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], **kw)
    dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], **kw)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check_workload(case, reruns=0):
    """fwd + bwd on the GPU, every output against the oracle; ``reruns`` more
    GPU runs must reproduce every output bit for bit."""
    import torch
    print(f"[workload] {case.name}", flush=True)
    host, dev, f64 = device_inputs(case)
    got = run_fwd_bwd(case, dev)
    for r in range(reruns):
        again = run_fwd_bwd(case, dev)
        torch.cuda.synchronize()
        for name in got:
            assert torch.equal(bits(got[name]), bits(again[name])), f"{case.name}: {name} differs on rerun {r + 1}"
        del again
    torch.cuda.synchronize()
    ref = oracle_full(case, f64)
    compare_all(case, got, ref)
    if case.kv_lens is not None:
        lens = np.clip(np.asarray(case.kv_lens), 0, case.Tkv)
        gdk, gdv, gdq = to_host64(got["dk"]), to_host64(got["dv"]), to_host64(got["dq"])
        for b, n in enumerate(lens):
            assert np.all(gdk[b, n:] == 0.0) and np.all(gdv[b, n:] == 0.0)
            if n == 0:
                assert np.all(to_host64(got["o"])[b] == 0.0) and np.all(gdq[b] == 0.0)
    return got


def test_fp32_correctness_workload_full():
    (case,) = workload_cases(0)
    check_workload(case, reruns=1)


@pytest.mark.parametrize("case", workload_cases(1), ids=lambda c: c.name)
def test_bf16_d64_grid_full(case):
    check_workload(case)


@pytest.mark.slow
@pytest.mark.parametrize("case", workload_cases(2), ids=lambda c: c.name)
def test_headline_T8192_full_and_bitwise_rerun(case):
    check_workload(case, reruns=1)


def test_kv_length_workload_full():
    (case,) = workload_cases(3)
    got = check_workload(case)
    # Batch 0 has a single valid key: the exact dQ and dK are zero there
    # (the pages report how far approximate exponentials move them).
    assert float(np.abs(to_host64(got["dq"][0])).max()) <= 1e-3
    assert float(np.abs(to_host64(got["dk"][0])).max()) <= 1e-3


@pytest.mark.parametrize("case", [
    Case("kvlen_out_of_range_d128_gqa", 3, 200, 300, 8, 2, 128, kv_lens=(-3, 350, 299), workload_id=130),
    Case("kvlen_out_of_range_d64_causal", 2, 333, 333, 4, 4, 64, causal=True, kv_lens=(333 + 50, -1),
         workload_id=131),
    Case("kvlen_out_of_range_fp32", 2, 70, 90, 2, 1, 64, "fp32", kv_lens=(-7, 1000), workload_id=132),
], ids=lambda c: c.name)
def test_kv_lengths_outside_range_are_clamped(case):
    """KV lengths below 0 or above Tkv act as 0 and Tkv (the header's clamp):
    the oracle clamps the same way."""
    check_workload(case)


def test_decode_kv_lengths_outside_range_are_clamped():
    from test_gpu_decode import check_decode
    check_decode(Case("dec_kvlen_out_of_range", 3, 4, 700, 8, 2, 128, kv_lens=(-5, 700 + 50, 1), workload_id=133,
                      decode=True))
