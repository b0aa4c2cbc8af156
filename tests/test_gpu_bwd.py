"""Backward parity of the HIP kernels against the float64 oracle on small and
ragged shapes, determinism and the split passes (needs an MI355X); the five
workloads are compared in full in test_gpu_workloads.py."""

import numpy as np
import pytest

import oracle
from forward_backward_amd.inputs import Case
from helpers import TOL, ZERO_TOL, device_inputs, rel_err, to_host64
from test_gpu_fwd import SMALL

pytestmark = pytest.mark.gpu


def run_fwd_bwd(case, dev):
    from forward_backward_amd import attn
    o, lse = attn.fwd(dev["q"], dev["k"], dev["v"], scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"],
                      window=case.window)
    dq, dk, dv = attn.bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], scale=case.scale, causal=case.causal,
                          kv_lens=dev["kv_lens"], window=case.window)
    return o, lse, dq, dk, dv


def check_bwd(case, zero_tol=ZERO_TOL):
    """Forward and backward on the GPU, dQ, dK and dV of every head against the oracle.
    ``zero_tol``: the absolute bound on a gradient whose exact value is zero everywhere."""
    import torch
    host, dev, f64 = device_inputs(case)
    print(f"[bwd] {case.name}", flush=True)
    _, _, dq, dk, dv = run_fwd_bwd(case, dev)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attention_bwd(f64["q"], f64["k"], f64["v"], f64["do"], case.scale, case.causal,
                                         f64["kv_lens"], window=case.window)
    gdq, gdk, gdv = to_host64(dq), to_host64(dk), to_host64(dv)
    pairs = {"dq": (gdq, rdq), "dk": (gdk, rdk), "dv": (gdv, rdv)}
    for name, (g, r) in pairs.items():
        err = rel_err(g, r, zero_tol)
        print(f"    {name} rel err {err:.3e} (max|got| {np.abs(g).max() if g.size else 0:.3e})", flush=True)
        assert err <= TOL[case.dtype], f"{case.name}: {name} rel err {err:.3e}"
    if case.kv_lens is not None:
        for b, n in enumerate(case.kv_lens):
            assert np.all(gdk[b, n:] == 0.0) and np.all(gdv[b, n:] == 0.0)
            if n == 0:
                assert np.all(gdq[b] == 0.0)
    return dq, dk, dv


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c.name)
def test_bwd_small(case):
    check_bwd(case)


def test_bwd_is_bitwise_deterministic():
    import torch
    case = Case("d128_T333_causal_gqa_kvlen", 2, 333, 333, 8, 2, 128, causal=True, kv_lens=(333, 200),
                workload_id=120)
    host, dev, _ = device_inputs(case)
    runs = [run_fwd_bwd(case, dev) for _ in range(3)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("case", [
    # B * Hkv * ceil(Tkv / 128) = 6 < 256: dK/dV splits the group's query heads
    # and writes fp32 partials into the workspace that dQ reads from too.
    Case("streams_d128_gqa_split_causal_kvlen", 1, 300, 300, 8, 2, 128, causal=True, kv_lens=(250,),
         workload_id=121),
    Case("streams_d64_window", 2, 500, 500, 4, 4, 64, window=(60, 10), workload_id=122),
], ids=lambda c: c.name)
def test_dkdv_and_dq_on_two_streams_match_the_sequential_call(case):
    """The dK/dV and dQ passes only read what the pre-pass wrote, so a caller
    may run them concurrently on two streams; the result must be the
    sequential call's, bit for bit."""
    import torch
    from forward_backward_amd import attn
    host, dev, _ = device_inputs(case)
    print(f"[bwd two streams] {case.name}", flush=True)
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = attn.fwd(q, k, v, **kw)
    dq_ref, dk_ref, dv_ref = attn.bwd(q, k, v, o, lse, do, **kw)
    ws = attn.bwd_workspace(q, k, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    attn.bwd_preprocess(o, lse, do, ws, q, k, **kw)
    ready = torch.cuda.Event()
    ready.record()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        s1.wait_event(ready)
        attn.bwd_dkdv(q, k, v, lse, do, ws, dk, dv, **kw)
    with torch.cuda.stream(s2):
        s2.wait_event(ready)
        attn.bwd_dq(q, k, v, lse, do, ws, dq, **kw)
    torch.cuda.synchronize()
    for got, ref in ((dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("case", [
    # 32 query heads on one KV head: the dK/dV head split runs 32 ways
    # (B * Hkv * ceil(Tkv / 128) = 2 workgroups without it) and the
    # reduction sums 32 fp32 partials per element.
    Case("gqa32_split32_d128_T200", 1, 200, 200, 32, 1, 128, workload_id=123),
    Case("gqa16_d64_T333_causal_kvlen", 2, 333, 333, 16, 1, 64, causal=True, kv_lens=(333, 129), workload_id=124),
    Case("gqa16_d256_T130_kvlen", 1, 130, 130, 16, 1, 256, kv_lens=(77,), workload_id=125),
    # Many short problems: 16 sequences of 64 tokens.
    Case("b16_d128_T64", 16, 64, 64, 4, 2, 128, workload_id=126),
], ids=lambda c: c.name)
def test_bwd_wide_groups_and_many_short_sequences(case):
    check_bwd(case)


@pytest.mark.parametrize("case", [
    # Some KV tiles past the lengths (a batch of length 0): items without query
    # rows are taken from the queue and stored as zeros.
    Case("queue_d128_gqa_causal_kvlen", 3, 700, 700, 8, 2, 128, causal=True, kv_lens=(700, 0, 333), workload_id=127),
    Case("queue_d128_T2048_window", 2, 2048, 2048, 4, 4, 128, causal=True, window=(300, 0), workload_id=128),
], ids=lambda c: c.name)
def test_dkdv_pass_repeats_and_graph_replays(case):
    """The head_dim-128 dK/dV pass hands out its work through counters in the
    workspace that the pre-pass zeroes and the pass leaves at zero: the pass
    repeated without the pre-pass, and a captured backward replayed with
    other work in between, give the eager call's gradients bit for bit."""
    import torch
    from forward_backward_amd import attn
    host, dev, _ = device_inputs(case)
    print(f"[dkdv repeats] {case.name}", flush=True)
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = attn.fwd(q, k, v, **kw)
    dq_ref, dk_ref, dv_ref = attn.bwd(q, k, v, o, lse, do, **kw)
    ws = attn.bwd_workspace(q, k, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    attn.bwd_preprocess(o, lse, do, ws, q, k, **kw)
    for _ in range(3):
        dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
        attn.bwd_dkdv(q, k, v, lse, do, ws, dk, dv, **kw)
        torch.cuda.synchronize()
        assert torch.equal(dk.view(torch.int16), dk_ref.view(torch.int16))
        assert torch.equal(dv.view(torch.int16), dv_ref.view(torch.int16))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            out = attn.bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        attn.bwd(q, k, v, o, lse, do, **kw)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(out, (dq_ref, dk_ref, dv_ref)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("case", [
    # 512 one-tile items (64 query rows, one query head per KV head) for 256
    # persistent workgroups: each workgroup chains several, and every item's
    # second tile is the next item's first.
    Case("queue_d128_one_tile_items", 64, 64, 64, 8, 8, 128, workload_id=134),
    # 480 items of 1, 3 and 5 tiles (causal, three 128-key tiles per head),
    # KV lengths that leave whole items empty in some batches.
    Case("queue_d128_mixed_item_lengths", 40, 300, 300, 4, 4, 128, causal=True,
         kv_lens=tuple((300, 60, 0, 211, 129)[b % 5] for b in range(40)), workload_id=135),
], ids=lambda c: c.name)
def test_dkdv_queue_item_mixes(case):
    """The head_dim-128 dK/dV workgroups take more items than there are
    workgroups: one-tile items, empty items and items of different lengths
    follow each other in one workgroup's stream of tiles."""
    check_bwd(case)


@pytest.mark.parametrize("case", [
    Case("dqpre_d128_gqa_causal_kvlen", 2, 333, 333, 8, 2, 128, causal=True, kv_lens=(333, 0), workload_id=136),
    Case("dqpre_d64_window_ragged", 2, 300, 300, 4, 4, 64, causal=True, window=(40, 0), workload_id=137),
    Case("dqpre_d32_unfused", 1, 200, 200, 4, 2, 32, workload_id=138),
], ids=lambda c: c.name)
def test_dq_and_preprocess_writes_the_preprocess_bits(case):
    """attn_bwd_dq_and_preprocess (at bf16 head_dim 64/128 one dQ launch that
    forms D itself) leaves the same workspace statistics (D, LSE * log2(e),
    the row terms) and the same dQ as the preprocess pass followed by dQ,
    bit for bit, including rows with no valid key (LSE = -inf)."""
    import torch
    from forward_backward_amd import attn
    host, dev, _ = device_inputs(case)
    print(f"[dq and preprocess] {case.name}", flush=True)
    kw = dict(scale=case.scale, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o, lse = attn.fwd(q, k, v, **kw)
    ws1 = attn.bwd_workspace(q, k, causal=case.causal, kv_lens=dev["kv_lens"], window=case.window)
    ws2 = torch.full_like(ws1, 0x5A)
    dq1, dq2 = torch.empty_like(q), torch.empty_like(q)
    attn.bwd_preprocess(o, lse, do, ws1, q, k, **kw)
    attn.bwd_dq(q, k, v, lse, do, ws1, dq1, **kw)
    attn.bwd_dq_and_preprocess(q, k, v, o, lse, do, ws2, dq2, **kw)
    torch.cuda.synchronize()
    # Workspace layout: D and LSE * log2(e) (fp32 per row), then 16 bytes of
    # row terms per row, each region starting on a 256-byte boundary.
    rows = case.B * case.Hq * case.Tq
    region = (rows * 4 + 255) // 256 * 256
    for name, lo, n in (("D", 0, rows * 4), ("LSE * log2(e)", region, rows * 4), ("row terms", 2 * region, rows * 16)):
        assert torch.equal(ws1[lo:lo + n], ws2[lo:lo + n]), name
    assert torch.equal(dq1.view(torch.int16), dq2.view(torch.int16))
