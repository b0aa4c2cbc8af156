"""Shared helpers of the GPU parity tests: transfers, error metric, tolerances."""

import numpy as np

from forward_backward_amd import inputs as I

# Tolerances of the metric max|a - b| / max|b| per output tensor.
TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = 1e-4


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(a))) if a.size else 0.0
    return float(np.max(np.abs(a - b)) / den)


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "fp32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    elif dtype == "int32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.cuda()


def to_host64(t):
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return I.bf16_bits_to_f32(bits).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def check_lse(gpu_lse, ref_lse, tol=LSE_TOL):
    """-inf exactly where the oracle has -inf; elsewhere the relative metric."""
    g = np.asarray(gpu_lse, dtype=np.float64)
    r = np.asarray(ref_lse, dtype=np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), "LSE -inf positions differ"
    fin = np.isfinite(r)
    if fin.any():
        err = rel_err(g[fin], r[fin])
        assert err <= tol, f"LSE rel err {err:.3e} > {tol}"


def device_inputs(case, seed=0, with_do=True):
    """Host arrays (storage format), device tensors and float64 copies for the oracle."""
    host = I.make_inputs(case, seed=seed, with_do=with_do)
    dev = {k: to_device(v, case.dtype) for k, v in host.items() if k != "kv_lens"}
    dev["kv_lens"] = None if host["kv_lens"] is None else to_device(host["kv_lens"], "int32")
    f64 = {k: I.to_float64(v, case.dtype) for k, v in host.items() if k != "kv_lens"}
    f64["kv_lens"] = host["kv_lens"]
    return host, dev, f64
