"""attn_decode_noalloc against attn_decode (needs an MI355X).

The allocation-free decode runs the same kernels on the library's static
scratch instead of a caller's workspace, so its outputs must equal
attn_decode's bit for bit. Two calls in a row, the second on a smaller
problem, check that the scratch left by one call does not leak into the next.
"""

import numpy as np
import pytest

from forward_backward_amd.inputs import Case, workload_cases
from helpers import TOL, device_inputs, rel_err, to_host64

pytestmark = pytest.mark.gpu

CASES = [
    workload_cases(4)[0],  # B4, 32 query heads over 8 KV heads, 16 queries, 16384-key cache, lengths per batch
    Case("noalloc_small_q5_g4_kv3000", 2, 5, 3000, 8, 2, 128, kv_lens=(1, 2999), workload_id=600, decode=True),
]


def test_noalloc_decode_equals_decode_on_two_calls_in_a_row():
    import torch
    from forward_backward_amd import attn
    for case in CASES:
        print(f"[noalloc decode] {case.name}", flush=True)
        host, dev, _ = device_inputs(case, with_do=False)
        q, k, v, lens = dev["q"], dev["k"], dev["v"], dev["kv_lens"]
        o = torch.empty_like(q)
        lse = torch.empty((case.B, case.Hq, case.Tq), dtype=torch.float32, device=q.device)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        attn.decode_noalloc(q, k, v, kv_lens=lens, scale=case.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        o_ref, lse_ref = attn.decode(q, k, v, kv_lens=lens, scale=case.scale)
        torch.cuda.synchronize()
        err = rel_err(to_host64(o), to_host64(o_ref))
        assert err <= TOL["bf16"], f"{case.name}: O differs from attn_decode by {err:.3e}"
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{case.name}: O not bit-identical"
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), f"{case.name}: LSE not bit-identical"
        assert np.isfinite(to_host64(o)).all()
