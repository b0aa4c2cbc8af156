"""head_dim 32 (bf16): forward, backward and decode parity against the float64 oracle (needs an MI355X).

The pages name head_dim 32 as a weak spot of the tuned kernels there ("H100
(Hopper)", known issues); here every bf16 kernel is instantiated for it, with
an LDS swizzle for 64-byte rows.
"""

import pytest

from forward_backward_amd.inputs import Case
from helpers import device_inputs
from test_gpu_bwd import check_bwd, run_fwd_bwd
from test_gpu_decode import check_decode
from test_gpu_fwd import check_case

pytestmark = pytest.mark.gpu

CASES = [
    Case("d32_T1", 2, 1, 1, 2, 2, 32, workload_id=400),
    Case("d32_T65_causal", 2, 65, 65, 4, 2, 32, causal=True, workload_id=401),
    Case("d32_T200_kvlen_gqa", 2, 200, 200, 8, 2, 32, kv_lens=(150, 0), workload_id=402),
    Case("d32_q130_kv300", 2, 130, 300, 4, 4, 32, workload_id=403),
    Case("d32_T333_window", 1, 333, 333, 4, 1, 32, window=(50, 10), workload_id=404),
    Case("d32_T1500_causal_gqa", 2, 1500, 1500, 8, 4, 32, causal=True, workload_id=405),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_d32_fwd(case):
    check_case(case)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_d32_bwd(case):
    check_bwd(case)


def test_d32_B4_H8_T2048_full():
    from test_gpu_workloads import check_workload
    check_workload(Case("d32_B4_H8_T2048", 4, 2048, 2048, 8, 8, 32, workload_id=406))


@pytest.mark.parametrize("case", [
    Case("d32_dec_q16_g4", 2, 16, 3000, 8, 2, 32, kv_lens=(3000, 1), workload_id=407, decode=True),
    Case("d32_dec_q1_g1", 3, 1, 5000, 4, 4, 32, kv_len_range=(0, 5000), workload_id=408, decode=True),
], ids=lambda c: c.name)
def test_d32_decode(case):
    check_decode(case)


def test_d32_is_bitwise_deterministic():
    import torch
    case = CASES[5]
    host, dev, _ = device_inputs(case)
    runs = [run_fwd_bwd(case, dev) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
