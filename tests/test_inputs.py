"""Seeded generator and host accounting (CPU only)."""

import os

import numpy as np
import pytest

from forward_backward_amd import inputs as I
from forward_backward_amd.metrics import attention_flops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    cases = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, 1 + 2.0**-8 + 2.0**-20, -(1 + 2.0**-8), 1 + 2.0**-9,
                      3.0e38, -0.0, np.inf, 1e-40], dtype=np.float32)
    bits = I.f32_to_bf16_bits(cases)
    back = I.bf16_bits_to_f32(bits)
    assert back[0] == one                       # tie -> even (mantissa 0)
    assert back[1] == np.float32(1 + 4 * 2.0**-8)  # tie -> even (rounds up)
    assert back[2] == np.float32(1 + 2 * 2.0**-8)  # above the tie -> up
    assert back[3] == -one
    assert back[4] == one
    assert np.isfinite(back[5]) and back[5] > 2.9e38
    assert bits[6] == 0x8000 and np.isinf(back[7])
    nan = I.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(I.bf16_bits_to_f32(nan))[0]


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    ours = I.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_generator_is_deterministic_and_tensors_differ():
    case = I.workload_cases(1)[0].replace(Tq=64, Tkv=64)
    a = I.make_inputs(case, seed=0)
    b = I.make_inputs(case, seed=0)
    c = I.make_inputs(case, seed=1)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == np.uint16 and np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert not np.array_equal(a["q"], a["k"])
    x = I.to_float64(a["q"], "bf16")
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05


def test_workloads_shapes_and_kv_lens():
    (c1,) = I.workload_cases(0)
    assert (c1.B, c1.Tq, c1.Hq, c1.D, c1.dtype) == (1, 128, 2, 64, "fp32") and c1.scale == 1 / 8
    assert len(I.workload_cases(1)) == 12
    assert {c.Tq for c in I.workload_cases(1)} == {512, 1024, 2048, 600, 1500, 3000}
    (c4,) = I.workload_cases(3)
    assert list(I.draw_kv_lens(c4)) == [1, 777, 2500, 4096]
    (c5,) = I.workload_cases(4)
    lens = I.draw_kv_lens(c5)
    assert lens.dtype == np.int32 and lens.shape == (4,)
    assert np.all((lens >= 1024) & (lens <= 16384))
    assert np.array_equal(lens, I.draw_kv_lens(c5))
    x = I.make_inputs(c1, with_do=False)
    assert x["q"].dtype == np.float32 and "do" not in x


def test_flop_convention_reproduces_pages_records():
    n = 0
    with open(os.path.join(GOLDEN, "flop_convention.tsv")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            impl, dtype, b, h, d, t, causal, mode, ms, tflops = line.rstrip("\n").split("\t")
            fl = attention_flops(int(b), int(h), int(t), int(t), int(d), bool(int(causal)), mode)
            ours = fl / (float(ms) * 1e-3) / 1e12
            assert abs(ours - float(tflops)) <= 1e-9 * float(tflops), line
            n += 1
    assert n == 317


def test_visible_pairs_counts_the_oracle_mask():
    """The work count the benchmark uses for masked workloads equals the number
    of True entries of the oracle's mask."""
    import oracle
    from forward_backward_amd.metrics import visible_pairs
    for t, causal, window, kv_len in ((37, False, None, None), (37, True, None, 20), (50, False, (3, 5), None),
                                      (50, True, (7, -1), 44), (64, False, (-1, 0), None), (9, False, (0, 0), 4)):
        n = t if kv_len is None else kv_len
        assert visible_pairs(t, t, causal, window, kv_len) == int(oracle.valid_mask(t, t, causal, n, window).sum())
