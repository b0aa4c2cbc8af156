"""Shared helpers of the GPU parity tests: transfers, error metric, tolerances,
and the whole-tensor oracle evaluation of a problem."""

import concurrent.futures
import os

import numpy as np

import oracle
from forward_backward_amd import inputs as I

# Tolerances of the metric max|a - b| / max|b| per output tensor.
TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = 1e-4


# Where the reference tensor is exactly zero the relative metric is undefined;
# the result must then be zero up to this absolute bound.
ZERO_TOL = 1e-6
# The one exception: when every query row sees exactly one key, the exact dQ
# and dK vanish (dP - D is zero), and what the bf16 kernels leave is the
# rounding difference between dP from the matrix product and D from the
# rounded O, scaled by K. The pages report such residue (about 1e-5 for a
# Triton kernel, 1e-1 for an approximate exponential; "H100 (Hopper)",
# section "Mosaic GPU"); the bound there is 1e-3 absolute.
SINGLE_KEY_TOL = 1e-3


def rel_err(a, b, zero_tol=ZERO_TOL):
    """max|a - b| / max|b| over the whole tensor ("GPU and CPU performance",
    section "Methodology"). When max|b| = 0 the check becomes
    max|a| <= zero_tol: the metric is 0 if that holds and infinite otherwise."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shapes differ: {a.shape} and {b.shape}")
    if not a.size:
        return 0.0
    den = float(np.max(np.abs(b)))
    if den == 0.0:
        return 0.0 if float(np.max(np.abs(a))) <= zero_tol else float("inf")
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


def _oracle_workers(tq, tkv):
    """Threads for the per-head oracle calls: the host's CPU share (at most 16,
    the share of one GPU), fewer when the score matrices would not fit in
    the free memory (about a dozen float64 [Tq, Tkv] arrays per call)."""
    cpus = min(16, len(os.sched_getaffinity(0)))
    try:
        import psutil
        free = psutil.virtual_memory().available
    except ImportError:  # pragma: no cover
        free = 16 << 30
    per_call = 12 * 8 * max(tq, 1) * max(tkv, 1) + (64 << 20)
    return max(1, min(cpus, int(0.6 * free) // per_call))


def oracle_full(case, f64, fwd=True, bwd=True):
    """The oracle's O, LSE (forward) and dQ, dK, dV (backward) of every head.

    The oracle is called once per (batch, query head) for the forward and
    once per (batch, KV head) with its G query heads for the backward, on
    slices of the inputs, from a thread pool with one BLAS thread per call
    (NumPy releases the interpreter lock inside its array operations). The
    results are those of one whole-tensor call; only the wall time differs.
    """
    from threadpoolctl import threadpool_limits

    q, k, v = f64["q"], f64["k"], f64["v"]
    B, Tq, Hq, D = q.shape
    Tkv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    lens = f64["kv_lens"]
    kw = dict(window=case.window)
    out = {}
    if fwd:
        out["o"] = np.empty(q.shape)
        out["lse"] = np.empty((B, Hq, Tq))
    if bwd:
        out["dq"] = np.empty(q.shape)
        out["dk"] = np.empty(k.shape)
        out["dv"] = np.empty(k.shape)

    def lens_of(b):
        return None if lens is None else np.asarray(lens[b:b + 1])

    def fwd_task(b, h):
        kh = h // G
        o, lse = oracle.attention_fwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, kh:kh + 1], v[b:b + 1, :, kh:kh + 1],
                                      case.scale, case.causal, lens_of(b), **kw)
        out["o"][b, :, h] = o[0, :, 0]
        out["lse"][b, h] = lse[0, 0]

    def bwd_task(b, kh):
        hs = slice(kh * G, (kh + 1) * G)
        dq, dk, dv = oracle.attention_bwd(q[b:b + 1, :, hs], k[b:b + 1, :, kh:kh + 1], v[b:b + 1, :, kh:kh + 1],
                                          f64["do"][b:b + 1, :, hs], case.scale, case.causal, lens_of(b), **kw)
        out["dq"][b, :, hs] = dq[0]
        out["dk"][b, :, kh] = dk[0, :, 0]
        out["dv"][b, :, kh] = dv[0, :, 0]

    tasks = []
    if fwd:
        tasks += [(fwd_task, b, h) for b in range(B) for h in range(Hq)]
    if bwd:
        tasks += [(bwd_task, b, kh) for b in range(B) for kh in range(Hkv)]
    workers = _oracle_workers(Tq, Tkv)
    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(fn, *args) for fn, *args in tasks]:
                f.result()
    return out


def compare_all(case, got, ref, label=""):
    """Every output of ``got`` (device tensors) against the oracle's, whole tensors.

    Returns the errors; asserts the bf16/fp32 bound on O, dQ, dK, dV and the
    LSE rule (-inf positions equal, relative error <= 1e-4 elsewhere)."""
    errs = {}
    for name in ("o", "dq", "dk", "dv"):
        if name in got and name in ref:
            errs[name] = rel_err(to_host64(got[name]), ref[name])
    if "lse" in got and "lse" in ref:
        g = to_host64(got["lse"])
        check_lse(g, ref["lse"])
        fin = np.isfinite(ref["lse"])
        errs["lse"] = rel_err(g[fin], ref["lse"][fin]) if fin.any() else 0.0
    print(f"    {label or case.name}: " + ", ".join(f"{n} {e:.3e}" for n, e in errs.items()), flush=True)
    for name, e in errs.items():
        bound = LSE_TOL if name == "lse" else TOL[case.dtype]
        assert e <= bound, f"{label or case.name}: {name} rel err {e:.3e} > {bound}"
    return errs
