"""head_dim 256 (bf16): forward, backward and decode parity against the float64 oracle (needs an MI355X).

The pages report head_dim 256 as a configuration whose tiles overflowed the
shared memory of the GPU there ("H100 (Hopper)", known issues). Here the
forward splits each query block over a pair of waves by role (S and softmax;
O), dQ runs one workgroup per compute unit, and dK/dV splits
each 32-key block over a pair of waves by role (one holds K and dV, the other
V and dK), two pairs per workgroup, with Q and dO in 32-row tiles.
"""

import pytest

from forward_backward_amd.inputs import Case
from helpers import device_inputs
from test_gpu_bwd import check_bwd, run_fwd_bwd
from test_gpu_decode import check_decode
from test_gpu_fwd import check_case

pytestmark = pytest.mark.gpu

CASES = [
    Case("d256_T1", 2, 1, 1, 2, 2, 256, workload_id=500),
    Case("d256_T65_causal", 2, 65, 65, 4, 4, 256, causal=True, workload_id=501),
    # B * Hkv * ceil(Tkv/128) = 4 < 256: the query heads of a group split over
    # workgroups (fp32 partials of whole rows, summed in split order)
    Case("d256_T200_kvlen_gqa_split", 2, 200, 200, 8, 2, 256, kv_lens=(150, 0), workload_id=502),
    Case("d256_q130_kv300", 2, 130, 300, 4, 4, 256, workload_id=503),
    Case("d256_T333_window_causal", 1, 333, 333, 4, 1, 256, causal=True, window=(70, -1), workload_id=504),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_d256_fwd(case):
    check_case(case)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_d256_bwd(case):
    check_bwd(case)


def test_d256_B2_H16_T2048_full():
    # 2 * 16 * 16 = 512 dK/dV workgroups: no head split; all passes at full tiles
    from test_gpu_workloads import check_workload
    check_workload(Case("d256_B2_H16_T2048", 2, 2048, 2048, 16, 16, 256, workload_id=505))


@pytest.mark.parametrize("case", [
    Case("d256_dec_q16_g4", 2, 16, 3000, 8, 2, 256, kv_lens=(3000, 1), workload_id=506, decode=True),
    Case("d256_dec_q1_g1", 3, 1, 5000, 4, 4, 256, kv_len_range=(0, 5000), workload_id=507, decode=True),
], ids=lambda c: c.name)
def test_d256_decode(case):
    check_decode(case)


def test_d256_is_bitwise_deterministic():
    import torch
    case = CASES[2]
    host, dev, _ = device_inputs(case)
    runs = [run_fwd_bwd(case, dev) for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
