"""Parity at the shapes of the pages' GQA and decode suites (needs an MI355X).

GQA suite: 32 query heads over 8 KV heads, head_dim 128, batch 1,
Lq = Lkv = T. Decode suite: one query per sequence, 32 query heads,
head_dim 128, 8 or 32 KV heads, full caches.
"""

import numpy as np
import pytest

from forward_backward_amd.inputs import workload_cases
from helpers import TOL, check_lse, device_inputs, rel_err, to_host64
from test_gpu_bwd import run_fwd_bwd
from test_gpu_decode import check_decode

pytestmark = pytest.mark.gpu

GQA = {c.Tq: c for c in workload_cases(5)}
DECODE = {(c.B, c.Tkv, c.Hkv): c for c in workload_cases(6)}


@pytest.mark.parametrize("T", [2048, 4096])
def test_gqa_suite_fwd_bwd_full(T):
    from test_gpu_workloads import check_workload
    check_workload(GQA[T])


def test_gqa_suite_native_equals_repeated_kv():
    """Native GQA (query head h reads KV head h // G) against the same problem
    run as multi-head attention on K/V repeated G times, with dK/dV summed over
    each group: both compute the same function, so they agree to rounding."""
    import torch
    from forward_backward_amd import attn
    case = GQA[1024]
    G = case.Hq // case.Hkv
    host, dev, _ = device_inputs(case)
    print(f"[gqa vs repeated] {case.name}", flush=True)
    o, lse, dq, dk, dv = run_fwd_bwd(case, dev)
    kr = dev["k"].repeat_interleave(G, dim=2).contiguous()
    vr = dev["v"].repeat_interleave(G, dim=2).contiguous()
    o2, lse2 = attn.fwd(dev["q"], kr, vr, scale=case.scale)
    dq2, dkr, dvr = attn.bwd(dev["q"], kr, vr, o2, lse2, dev["do"], scale=case.scale)
    torch.cuda.synchronize()
    sh = (case.B, case.Tkv, case.Hkv, G, case.D)
    dk2 = to_host64(dkr).reshape(sh).sum(axis=3)
    dv2 = to_host64(dvr).reshape(sh).sum(axis=3)
    # The repeated run reads the same K/V rows in the same order for each
    # query head, so O, LSE and dQ are identical bit for bit.
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(lse, lse2)
    assert torch.equal(dq.view(torch.int16), dq2.view(torch.int16))
    # dK/dV: the native kernel sums the group in fp32 and rounds once; the
    # repeated run rounds each head's gradient to bf16 before the sum.
    for name, a, b in (("dk", to_host64(dk), dk2), ("dv", to_host64(dv), dv2)):
        err = rel_err(a, b)
        print(f"    {name} native vs repeated rel err {err:.3e}", flush=True)
        assert err <= TOL["bf16"], f"{name}: {err:.3e}"


@pytest.mark.parametrize("key", [(8, 4096, 8), (8, 4096, 32), (1, 65536, 8)], ids=lambda k: f"B{k[0]}_kv{k[1]}_hkv{k[2]}")
def test_decode_suite(key):
    check_decode(DECODE[key])
