"""Forward parity of the HIP kernels against the float64 oracle on small and
ragged shapes (needs an MI355X); the five workloads are compared in full in
test_gpu_workloads.py."""

import numpy as np
import pytest

import oracle
from forward_backward_amd.inputs import Case
from helpers import TOL, check_lse, device_inputs, rel_err, to_host64

pytestmark = pytest.mark.gpu

SMALL = [
    Case("d64_T1", 2, 1, 1, 2, 2, 64, workload_id=100),
    Case("d64_T63_causal", 2, 63, 63, 4, 4, 64, causal=True, workload_id=101),
    Case("d64_T64", 2, 64, 64, 4, 4, 64, workload_id=102),
    Case("d64_T65_causal", 2, 65, 65, 4, 2, 64, causal=True, workload_id=103),
    Case("d64_T127", 2, 127, 127, 4, 4, 64, workload_id=104),
    Case("d64_T200_causal_kvlen", 2, 200, 200, 4, 4, 64, causal=True, kv_lens=(150, 37), workload_id=105),
    Case("d128_T200_gqa_kvlen", 2, 200, 200, 8, 2, 128, kv_lens=(150, 37), workload_id=106),
    Case("d128_T333_causal_gqa", 2, 333, 333, 4, 1, 128, causal=True, workload_id=107),
    Case("d128_q100_kv300_empty_rows", 2, 100, 300, 2, 2, 128, kv_lens=(0, 300), workload_id=108),
    Case("d128_q130_kv70_kvlen1", 3, 130, 70, 2, 1, 128, kv_lens=(1, 70, 64), workload_id=109),
    Case("d64_T700_full", 1, 700, 700, 2, 2, 64, workload_id=110),
    Case("fp32_d128_T100_causal", 2, 100, 100, 2, 1, 128, "fp32", causal=True, workload_id=111),
    Case("fp32_d64_kvlen", 2, 40, 90, 2, 2, 64, "fp32", kv_lens=(0, 77), workload_id=112),
]


def run_fwd(case, dev):
    from forward_backward_amd import attn
    return attn.fwd(dev["q"], dev["k"], dev["v"], scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"],
                    window=case.window)


def check_case(case):
    """Forward on the GPU, O and LSE of every head against the oracle."""
    import torch
    host, dev, f64 = device_inputs(case, with_do=False)
    print(f"[fwd] {case.name}", flush=True)
    o, lse = run_fwd(case, dev)
    torch.cuda.synchronize()
    ro, rlse = oracle.attention_fwd(f64["q"], f64["k"], f64["v"], case.scale, case.causal, f64["kv_lens"],
                                    window=case.window)
    go, glse = to_host64(o), to_host64(lse)
    err = rel_err(go, ro)
    assert err <= TOL[case.dtype], f"{case.name}: O rel err {err:.3e}"
    check_lse(glse, rlse)
    # rows without a valid key are exactly zero
    if case.kv_lens is not None:
        for b, n in enumerate(case.kv_lens):
            if n == 0:
                assert np.all(go[b] == 0.0) and np.all(np.isneginf(glse[b]))
    return o, lse, dev


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_fwd_small(case):
    check_case(case)


def test_fwd_is_deterministic():
    import torch
    case = SMALL[7]
    host, dev, _ = device_inputs(case, with_do=False)
    o1, l1 = run_fwd(case, dev)
    o2, l2 = run_fwd(case, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)

