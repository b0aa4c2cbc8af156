"""fp32 path on the fp32 matrix cores: parity with the float64 oracle (needs an MI355X).

The cases span several 64- and 128-row tiles with ragged tails at head_dim
32, 64 and 128, with causal masking, KV lengths (including 0 and 1), GQA,
Tq != Tkv and local windows, plus the pages' fp32 grid shape (batch 4, 8
heads, T = 4096) on sampled heads. Tolerance: max|a - b| / max|b| <= 1e-4.
"""

import pytest

from forward_backward_amd.inputs import Case, workload_cases
from helpers import device_inputs
from test_gpu_bwd import check_bwd, run_fwd_bwd
from test_gpu_fwd import check_case

pytestmark = pytest.mark.gpu

CASES = [
    Case("fp32_d32_T1", 2, 1, 1, 2, 2, 32, "fp32", workload_id=400),
    Case("fp32_d32_T200_causal", 2, 200, 200, 4, 2, 32, "fp32", causal=True, workload_id=401),
    Case("fp32_d64_T65", 2, 65, 65, 4, 4, 64, "fp32", workload_id=402),
    Case("fp32_d64_T333_causal_gqa", 2, 333, 333, 8, 2, 64, "fp32", causal=True, workload_id=403),
    Case("fp32_d128_T257_kvlen", 3, 257, 257, 4, 4, 128, "fp32", kv_lens=(0, 1, 200), workload_id=404),
    Case("fp32_d128_q70_kv300_gqa", 2, 70, 300, 8, 1, 128, "fp32", kv_lens=(299, 64), workload_id=405),
    Case("fp32_d128_q300_kv70", 1, 300, 70, 2, 2, 128, "fp32", workload_id=406),
    Case("fp32_d128_T500_causal", 1, 500, 500, 2, 1, 128, "fp32", causal=True, workload_id=407),
    Case("fp32_d64_T300_window", 2, 300, 300, 4, 2, 64, "fp32", window=(40, 17), workload_id=408),
    Case("fp32_d32_T700_causal_window_kvlen", 2, 700, 700, 2, 1, 32, "fp32", causal=True, window=(129, 0),
         kv_lens=(700, 301), workload_id=409),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_fp32_fwd(case):
    check_case(case)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_fp32_bwd(case):
    check_bwd(case)


SCALE = {c.name: c for c in workload_cases(8)}


@pytest.mark.parametrize("name", ["fp32_d128_T4096_full", "fp32_d64_T4096_causal"])
def test_fp32_grid_full(name):
    from test_gpu_workloads import check_workload
    check_workload(SCALE[name])


def test_fp32_is_deterministic():
    import torch
    case = CASES[3]
    host, dev, _ = device_inputs(case)
    print(f"[fp32 determinism] {case.name}", flush=True)
    r1 = run_fwd_bwd(case, dev)
    r2 = run_fwd_bwd(case, dev)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
