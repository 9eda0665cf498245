"""The seeded input generator (no GPU): one rounding from float64 into the
storage types, the integer and power-of-two recipes, and determinism."""
import numpy as np
import pytest

from oracle import oracle as oracle_mod
from sparse_attention_kv_ds_amd import synth


@pytest.fixture(scope="module")
def orc():
    if not __import__("os").path.exists(oracle_mod.LIB):
        oracle_mod.build()
    return oracle_mod.load()


def test_fp16_rounding_is_one_rounding_from_float64():
    """numpy converts float64 to float16 directly, with ties to even: the
    generator must agree on random values, on every midpoint between fp16
    neighbours and on values a hair either side (where rounding through
    float32 first would go wrong), and at the overflow threshold."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) / np.sqrt(128.0),
                        rng.standard_normal(20000) * 3e4, rng.standard_normal(20000) * 1e-6])
    with np.errstate(over="ignore"):  # (numpy's cast warns where it overflows to inf)
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(synth.to_bits(x, "f16"), want)
    v = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2
    for m in (mids, np.nextafter(mids, 0.0), np.nextafter(mids, np.inf), -mids):
        assert np.array_equal(synth.to_bits(m, "f16"), m.astype(np.float16).view(np.uint16))
    # above the largest midpoint below 2^16 by less than a float32 step: one
    # rounding keeps 65504, rounding through float32 first reaches the tie
    x = np.array([65519.999, 65520.0, 65536.0, -65520.0, 0.0, -0.0, np.inf, -np.inf])
    assert synth.to_bits(x, "f16").tolist() == [0x7BFF, 0x7C00, 0x7C00, 0xFC00, 0, 0x8000,
                                                0x7C00, 0xFC00]


def test_bf16_rounding_matches_the_oracle_encoder(orc):
    """bf16: against the oracle's own encoder (pinned by its round-trip and
    midpoint checks) on random values and on values a hair above and below
    bf16 midpoints, where a rounding through float32 would land on the tie."""
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) / np.sqrt(128.0), rng.standard_normal(2000) * 1e30])
    b = np.arange(0, 0x7F80, 97, dtype=np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    x = np.concatenate([x, mid, mid + (hi - lo) * 2.0 ** -20, mid - (hi - lo) * 2.0 ** -20])
    got = synth.to_bits(x, "bf16")
    want = np.array([orc.double_to_bf16(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_integer_recipe_and_determinism():
    d = synth.make("tiny")
    q = d["q"].view(np.float16).astype(np.float64)
    k = d["k"].view(np.float16).astype(np.float64)
    assert set(np.unique(q)) <= set(range(-4, 5)) and set(np.unique(k)) <= set(range(-4, 5))
    assert set(np.unique(np.abs(d["w"]))) <= {1.0, 0.5, 0.25, 0.125}
    e = synth.make("tiny")
    assert all(np.array_equal(d[x], e[x]) for x in ("q", "k", "w", "pos"))
    assert d["pos"].tolist() == list(range(256))
