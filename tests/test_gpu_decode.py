"""Split-KV decode parity against the float64 oracle (needs an MI355X)."""

import numpy as np
import pytest

import oracle
from forward_backward_amd.inputs import Case, workload_cases
from helpers import TOL, check_lse, device_inputs, rel_err, to_host64

pytestmark = pytest.mark.gpu

SMALL = [
    Case("dec_q1_g1_kv700", 2, 1, 700, 2, 2, 128, kv_lens=(700, 333), workload_id=200, decode=True),
    Case("dec_q16_g4_kv3000", 2, 16, 3000, 8, 2, 128, kv_lens=(1, 2999), workload_id=201, decode=True),
    Case("dec_q32_g4_rows128", 1, 32, 1500, 8, 2, 128, kv_lens=(1500,), workload_id=202, decode=True),
    Case("dec_d64_q5_g8", 2, 5, 2048, 16, 2, 64, kv_lens=(0, 2048), workload_id=203, decode=True),
    Case("dec_nomask_q3", 1, 3, 1100, 4, 4, 64, workload_id=204, decode=True),
    # more than 64 batches: the on-device range schedule works in chunks of 64
    Case("dec_b70_kvrange", 70, 1, 300, 2, 1, 64, kv_len_range=(0, 300), workload_id=205, decode=True),
    # packed rows over two row blocks (Tq * G = 80)
    Case("dec_q20_g4_two_rowblocks", 2, 20, 900, 8, 2, 128, kv_lens=(900, 77), workload_id=206, decode=True),
]


def run_decode(case, dev, num_splits=0):
    from forward_backward_amd import attn
    return attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale,
                       num_splits=num_splits)


def check_decode(case, num_splits=0):
    import torch
    host, dev, f64 = device_inputs(case, with_do=False)
    print(f"[decode] {case.name} splits={num_splits}", flush=True)
    o, lse = run_decode(case, dev, num_splits)
    torch.cuda.synchronize()
    ro, rlse = oracle.attention_decode(f64["q"], f64["k"], f64["v"], case.scale, f64["kv_lens"])
    go, glse = to_host64(o), to_host64(lse)
    err = rel_err(go, ro)
    assert err <= TOL["bf16"], f"{case.name}: O rel err {err:.3e}"
    check_lse(glse, rlse)
    if case.kv_lens is not None:
        for b, n in enumerate(case.kv_lens):
            if n == 0:
                assert np.all(go[b] == 0.0)
    return o, lse, dev


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_decode_small(case):
    check_decode(case)


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 1000])
def test_decode_split_count_changes_rounding_only(splits):
    check_decode(SMALL[1], num_splits=splits)


def test_decode_gqa_workload_full():
    (case,) = workload_cases(4)
    check_decode(case)


def test_decode_matches_forward_kernel():
    import torch
    from forward_backward_amd import attn
    case = SMALL[1]
    o, lse, dev = check_decode(case)
    of, lsef = attn.fwd(dev["q"], dev["k"], dev["v"], scale=case.scale, kv_lens=dev["kv_lens"])
    torch.cuda.synchronize()
    assert rel_err(to_host64(o), to_host64(of)) <= TOL["bf16"]
    check_lse(to_host64(lse), to_host64(lsef))


def test_decode_is_deterministic():
    import torch
    (case,) = workload_cases(4)
    host, dev, _ = device_inputs(case, with_do=False)
    a = run_decode(case, dev)
    b = run_decode(case, dev)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_decode_caches_past_2_31_elements():
    """Decode over K/V caches of 2^31 elements each (B = 64, 262144 keys, one KV
    head, head_dim 128, 4 query heads, KV lengths per batch). Three seeded
    batches repeat along the batch axis; they are checked against the oracle,
    and every batch must equal its source bit for bit (equal lengths give equal
    key ranges and the same combine order wherever the batch sits)."""
    import torch
    from forward_backward_amd import attn
    small = Case("big_dec_src_kv262144", 3, 1, 262144, 4, 1, 128, kv_lens=(262144, 1, 100000), workload_id=321,
                 decode=True)
    host, dev, f64 = device_inputs(small, with_do=False)
    B = 64
    print(f"[decode 2^31 elements] B={B} keys={small.Tkv}", flush=True)
    idx = torch.arange(B, device="cuda") % small.B
    q, k, v = (torch.index_select(dev[n], 0, idx).contiguous() for n in ("q", "k", "v"))
    assert k.numel() >= 2**31
    lens = torch.index_select(dev["kv_lens"], 0, idx).contiguous()
    o, lse = attn.decode(q, k, v, kv_lens=lens, scale=small.scale)
    torch.cuda.synchronize()
    for name, t, bits in (("o", o, o.view(torch.int16)), ("lse", lse, lse.view(torch.int32))):
        assert torch.equal(bits, torch.index_select(bits[:small.B], 0, idx)), f"{name}: a batch differs from its source"
    del k, v
    ro, rlse = oracle.attention_decode(f64["q"], f64["k"], f64["v"], small.scale, f64["kv_lens"])
    err = rel_err(to_host64(o[:small.B]), ro)
    print(f"    o rel err {err:.3e}", flush=True)
    assert err <= TOL["bf16"], f"O rel err {err:.3e}"
    check_lse(to_host64(lse[:small.B]), rlse)


@pytest.mark.parametrize("case", [
    Case("dec_all_lengths_zero", 3, 4, 500, 8, 2, 128, kv_lens=(0, 0, 0), workload_id=210, decode=True),
    Case("dec_empty_cache", 2, 3, 0, 4, 1, 64, workload_id=211, decode=True),
], ids=lambda c: c.name)
def test_decode_without_valid_keys_writes_zeros(case):
    """Segments with no valid key get no key range; the combine writes O = 0
    and LSE = -inf for every one of their rows."""
    import torch
    host, dev, _ = device_inputs(case, with_do=False)
    print(f"[decode empty] {case.name}", flush=True)
    o, lse = run_decode(case, dev)
    torch.cuda.synchronize()
    assert torch.all(o.float() == 0.0)
    assert torch.all(torch.isneginf(lse))


def test_decode_workspace_reuse():
    """One workspace serves calls of several shapes and split budgets: each
    result equals a call with a fresh workspace bit for bit."""
    import torch
    from forward_backward_amd import attn
    big = workload_cases(4)[0]
    host, dev, _ = device_inputs(big, with_do=False)
    ws = attn.decode_workspace(dev["q"], dev["k"], num_splits=1000)
    runs = [(big, 0), (SMALL[1], 1000), (SMALL[5], 0), (big, 7), (SMALL[6], 2), (big, 0)]
    for case, splits in runs:
        print(f"[decode workspace reuse] {case.name} splits={splits}", flush=True)
        _, d, _ = device_inputs(case, with_do=False)
        o, lse = attn.decode(d["q"], d["k"], d["v"], kv_lens=d["kv_lens"], scale=case.scale, num_splits=splits,
                             workspace=ws)
        o2, lse2 = attn.decode(d["q"], d["k"], d["v"], kv_lens=d["kv_lens"], scale=case.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def test_decode_one_workspace_over_new_inputs_and_many_calls():
    """With one workspace, calls on new inputs of the same shape each match
    the oracle (a combine that read a previous call's partials would not), and
    twenty calls on the same inputs give the same bits."""
    import torch
    from forward_backward_amd import attn
    case = SMALL[1]
    ws = None
    for seed in (0, 1, 2):
        host, dev, f64 = device_inputs(case, seed=seed, with_do=False)
        if ws is None:
            ws = attn.decode_workspace(dev["q"], dev["k"])
        print(f"[decode new inputs] {case.name} seed={seed}", flush=True)
        o, lse = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
        torch.cuda.synchronize()
        ro, rlse = oracle.attention_decode(f64["q"], f64["k"], f64["v"], case.scale, f64["kv_lens"])
        assert rel_err(to_host64(o), ro) <= TOL["bf16"]
        check_lse(to_host64(lse), rlse)
    (big,) = workload_cases(4)
    _, dev, _ = device_inputs(big, with_do=False)
    ws = attn.decode_workspace(dev["q"], dev["k"])
    ref = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=big.scale, workspace=ws)
    for it in range(20):
        o, lse = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=big.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), f"call {it}"
        assert torch.equal(lse.view(torch.int32), ref[1].view(torch.int32)), f"call {it}"


def test_decode_graph_replays():
    """Each replay of a captured decode call (with eager calls on the same
    workspace in between) equals the eager result bit for bit."""
    import torch
    from forward_backward_amd import attn
    (case,) = workload_cases(4)
    _, dev, _ = device_inputs(case, with_do=False)
    ws = attn.decode_workspace(dev["q"], dev["k"])
    ref = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        out = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(5):
        print(f"[decode graph] replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0].view(torch.int16), ref[0].view(torch.int16)), f"replay {rep}"
        assert torch.equal(out[1].view(torch.int32), ref[1].view(torch.int32)), f"replay {rep}"
        eager = attn.decode(dev["q"], dev["k"], dev["v"], kv_lens=dev["kv_lens"], scale=case.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager[0].view(torch.int16), ref[0].view(torch.int16))


@pytest.mark.parametrize("case,splits", [
    # 256 segments (64 batches x 4 KV heads, one row block): the automatic
    # split budget is 1, so the kernel writes the output itself; a quarter of
    # the batches have no valid key and get their rows from spare workgroups.
    (Case("dec_direct_b64_seg256", 64, 1, 1000, 16, 4, 128, kv_lens=tuple((0, 1, 640, 999)[b % 4] for b in range(64)),
          workload_id=220, decode=True), 0),
    (Case("dec_direct_d64_empty_batch", 2, 5, 2048, 16, 2, 64, kv_lens=(0, 2048), workload_id=203, decode=True), 1),
    (Case("dec_direct_empty_cache", 2, 3, 0, 4, 1, 64, workload_id=211, decode=True), 1),
], ids=lambda x: x.name if hasattr(x, "name") else f"splits{x}")
def test_decode_one_range_per_segment_writes_the_output(case, splits):
    """With a split budget of 1 every segment is one key range and the split
    kernel writes O and the LSE itself (no combine launch); rows of segments
    without keys come from the workgroups past the last range. Checked against
    the oracle, zero rows, and bit-for-bit reruns."""
    import torch
    from forward_backward_amd import attn
    if splits == 0:
        assert attn.decode_num_splits(case.B, case.Tq, case.Tkv, case.Hq, case.Hkv, case.D) == 1
    host, dev, f64 = device_inputs(case, with_do=False)
    print(f"[decode direct] {case.name} splits={splits}", flush=True)
    o, lse = run_decode(case, dev, splits)
    o2, lse2 = run_decode(case, dev, splits)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    go, glse = to_host64(o), to_host64(lse)
    lens = host["kv_lens"] if host["kv_lens"] is not None else np.full(case.B, case.Tkv)
    for b in range(case.B):
        if min(max(int(lens[b]), 0), case.Tkv) == 0:
            assert np.all(go[b] == 0.0) and np.all(np.isneginf(glse[b])), f"batch {b}"
    if case.Tkv == 0:
        return
    ro, rlse = oracle.attention_decode(f64["q"], f64["k"], f64["v"], case.scale, f64["kv_lens"])
    err = rel_err(go, ro)
    assert err <= TOL["bf16"], f"{case.name}: O rel err {err:.3e}"
    check_lse(glse, rlse)
