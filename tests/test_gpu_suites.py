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


# Every batch-1 shape of the decode suite, and batch 8 at 4096 keys, against
# the oracle on the whole output.
DIRECT = [k for k in sorted(DECODE) if k[0] == 1] + [(8, 4096, 8), (8, 4096, 32)]


@pytest.mark.parametrize("key", DIRECT, ids=lambda k: f"B{k[0]}_kv{k[1]}_hkv{k[2]}")
def test_decode_suite(key):
    check_decode(DECODE[key])


@pytest.mark.parametrize("n,hkv", [(16384, 8), (16384, 32), (65536, 8), (65536, 32)],
                         ids=lambda v: str(v))
def test_decode_suite_batch8_repeated(n, hkv):
    """Batch 8 of the decode suite at 16k and 64k keys, 32 query heads, one
    query each, full caches; 64k keys with 8 KV heads is the pages' decode
    peak point ("Attention performance", section "Grouped-query attention and
    decoding"). Two seeded batches are repeated along the batch axis on the
    device, so the host holds the oracle's inputs for two batches only; those
    two are checked against the oracle, and every batch must equal its source
    bit for bit (equal lengths give every batch the same key ranges and merge
    order)."""
    import torch
    from forward_backward_amd import attn
    from forward_backward_amd.inputs import Case
    wid = (610 if n == 65536 else 650) + hkv
    src = Case(f"dec_b8_src_kv{n}_hkv{hkv}", 2, 1, n, 32, hkv, 128, workload_id=wid, decode=True)
    host, dev, f64 = device_inputs(src, with_do=False)
    B = 8
    print(f"[decode batch 8, repeated sources] B{B} keys {src.Tkv} Hkv {hkv}", flush=True)
    idx = torch.arange(B, device="cuda") % src.B
    q, k, v = (torch.index_select(dev[n], 0, idx).contiguous() for n in ("q", "k", "v"))
    o, lse = attn.decode(q, k, v, scale=src.scale)
    torch.cuda.synchronize()
    for name, bits in (("o", o.view(torch.int16)), ("lse", lse.view(torch.int32))):
        assert torch.equal(bits, torch.index_select(bits[:src.B], 0, idx)), f"{name}: a batch differs from its source"
    del k, v
    from helpers import oracle_full
    ref = oracle_full(src, f64, bwd=False)
    err = rel_err(to_host64(o[:src.B]), ref["o"])
    print(f"    o rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    check_lse(to_host64(lse[:src.B]), ref["lse"])
