"""Local window masks: parity of the HIP kernels against the float64 oracle (needs an MI355X).

Key j is visible to query i iff i - left <= j <= i + right (negative = no
bound), combined by AND with the causal and KV-length masks. The cases cover
windows narrower than a tile, windows that start or end inside a tile,
one-sided windows, windows with causal masking and with KV lengths, GQA,
ragged lengths, both head dims and the fp32 path.
"""

import numpy as np
import pytest

from forward_backward_amd.inputs import Case
from helpers import SINGLE_KEY_TOL, ZERO_TOL, device_inputs, rel_err, to_host64
from test_gpu_bwd import check_bwd, run_fwd_bwd
from test_gpu_fwd import check_case

pytestmark = pytest.mark.gpu

CASES = [
    Case("win_d128_T300_l40_r40", 2, 300, 300, 4, 2, 128, window=(40, 40), workload_id=300),
    Case("win_d128_T700_l100_r0", 1, 700, 700, 4, 4, 128, window=(100, 0), workload_id=301),
    Case("win_d64_T513_l0_r70_kvlen", 2, 513, 513, 8, 2, 64, window=(0, 70), kv_lens=(513, 200), workload_id=302),
    Case("win_d128_T1000_l250_causal", 2, 1000, 1000, 4, 1, 128, causal=True, window=(250, -1), workload_id=303),
    Case("win_d64_T400_r5_onesided", 1, 400, 400, 2, 2, 64, window=(-1, 5), workload_id=304),
    Case("win_d128_T129_zero_width", 2, 129, 129, 2, 2, 128, window=(0, 0), workload_id=305),
    Case("win_d128_T640_l1_r1_kvlen0", 2, 640, 640, 4, 2, 128, window=(1, 1), kv_lens=(0, 333), workload_id=306),
    Case("win_fp32_d64_T90_l7_r3", 2, 90, 90, 2, 1, 64, "fp32", window=(7, 3), workload_id=307),
    Case("win_fp32_d128_T60_causal_l5", 1, 60, 60, 2, 2, 128, "fp32", causal=True, window=(5, 0), workload_id=308),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_window_fwd(case):
    check_case(case)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_window_bwd(case):
    # A zero-width window leaves every row one key: the exact dQ and dK are
    # zero everywhere and only the single-key absolute bound applies to them.
    single = case.window == (0, 0)
    _, dk, dv = check_bwd(case, zero_tol=SINGLE_KEY_TOL if single else ZERO_TOL)
    # Keys no query sees (past the KV length) get exactly zero gradients.
    if case.kv_lens is not None:
        gdk, gdv = to_host64(dk), to_host64(dv)
        for b, n in enumerate(case.kv_lens):
            assert np.all(gdk[b, n:] == 0.0) and np.all(gdv[b, n:] == 0.0)


def test_window_d128_T4096_full():
    """A long sequence with a 512-key band: most tiles are skipped on both sides."""
    from test_gpu_workloads import check_workload
    check_workload(Case("win_d128_T4096_l512_r64", 2, 4096, 4096, 8, 2, 128, window=(512, 64), workload_id=309))


def test_window_wider_than_sequence_equals_no_window():
    import torch
    from forward_backward_amd import attn
    case = Case("win_full_T333", 2, 333, 333, 4, 2, 128, causal=True, workload_id=310)
    host, dev, _ = device_inputs(case)
    plain = run_fwd_bwd(case, dev)
    wide = run_fwd_bwd(case.replace(window=(333, 1000)), dev)
    torch.cuda.synchronize()
    for a, b in zip(plain, wide):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    # A left bound of T with right bound 0 is the causal mask.
    causal = case.replace(causal=False, window=(333, 0))
    o2, lse2 = attn.fwd(dev["q"], dev["k"], dev["v"], scale=case.scale, window=causal.window)
    torch.cuda.synchronize()
    assert rel_err(to_host64(o2), to_host64(plain[0])) == 0.0


def test_window_is_bitwise_deterministic():
    import torch
    case = CASES[3]
    host, dev, _ = device_inputs(case)
    runs = [run_fwd_bwd(case, dev) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
