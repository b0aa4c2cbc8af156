"""The parity helpers themselves (CPU only): the threaded whole-tensor oracle
driver equals one whole-tensor oracle call, and the error metric follows its
definition, including the all-zero reference."""

import math

import numpy as np
import pytest

import oracle
from forward_backward_amd.inputs import Case
from helpers import ZERO_TOL, oracle_full, rel_err
from forward_backward_amd import inputs as I


@pytest.mark.parametrize("case", [
    Case("h_gqa_kvlen_window", 3, 40, 40, 6, 2, 8, causal=True, kv_lens=(40, 0, 17), window=(9, 3), workload_id=900),
    Case("h_plain_q_ne_kv", 2, 23, 31, 4, 4, 16, kv_lens=(-4, 99), workload_id=901),
    Case("h_fp32_gqa3", 1, 17, 17, 3, 1, 8, "fp32", workload_id=902),
], ids=lambda c: c.name)
def test_threaded_oracle_equals_whole_tensor_call(case):
    host = I.make_inputs(case)
    f64 = {k: I.to_float64(v, case.dtype) for k, v in host.items() if k != "kv_lens"}
    f64["kv_lens"] = host["kv_lens"]
    got = oracle_full(case, f64)
    o, lse = oracle.attention_fwd(f64["q"], f64["k"], f64["v"], case.scale, case.causal, f64["kv_lens"],
                                  window=case.window)
    dq, dk, dv = oracle.attention_bwd(f64["q"], f64["k"], f64["v"], f64["do"], case.scale, case.causal,
                                      f64["kv_lens"], window=case.window)
    for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert not np.isnan(got[name]).any(), name
        np.testing.assert_allclose(got[name], ref, rtol=0, atol=1e-12, err_msg=name)
    assert np.array_equal(np.isneginf(got["lse"]), np.isneginf(lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(got["lse"][fin], lse[fin], rtol=0, atol=1e-12)


def test_rel_err_definition():
    b = np.array([[1.0, -4.0], [2.0, 0.5]])
    a = b + np.array([[0.0, 0.02], [-0.04, 0.0]])
    assert rel_err(a, b) == pytest.approx(0.04 / 4.0)
    # All-zero reference: the result must be zero within the absolute bound.
    z = np.zeros((3, 2))
    assert rel_err(z, z) == 0.0
    assert rel_err(z + ZERO_TOL, z) == 0.0
    assert math.isinf(rel_err(z + 2 * ZERO_TOL, z))
    assert math.isinf(rel_err(z + 1e-3, z))  # would pass a 1e-2 bound as a plain max|a|
    with pytest.raises(ValueError):
        rel_err(np.zeros(3), np.zeros(4))
