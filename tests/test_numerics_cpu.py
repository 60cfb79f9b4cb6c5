"""Host-side checks of the arithmetic the kernels rely on (no GPU needed).

The gate projection for bf16 x splits each fp32 gate weight into three bf16 parts,
w = w1 + w2 + w3 with w1 = bf16(w), w2 = bf16(w - w1), w3 = w - w1 - w2, and claims the
split is exact (w3 is itself a bf16 value and the sum restores w bit for bit) for every
weight whose bf16 rounding stays finite (|w| below about 3.39e38) and that is not so
small that the third part underflows; and that a bf16 x times a bf16 part is exact in
fp32.  These are facts of the number formats,
checked here with numpy on the bit patterns: round-to-nearest-even fp32 -> bf16 written
out from its definition.
"""
import numpy as np


def bf16_rne(a):
    """fp32 -> bf16 (as fp32 values), round to nearest even."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def is_bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) & 0xFFFF) == 0


def split3(w):
    w = np.asarray(w, np.float32)
    w1 = bf16_rne(w)
    r = (w - w1).astype(np.float32)
    w2 = bf16_rne(r)
    w3 = (r - w2).astype(np.float32)
    return w1, w2, w3


def test_bf16_round_reference():
    # spot values: ties to even, and a carry into the exponent
    a = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, 2.0 - 2 ** -9], np.float32)
    assert bf16_rne(a).tolist() == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, 2.0]


def test_three_way_split_is_exact():
    rng = np.random.default_rng(0)
    w = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1 / 64),   # gate-like scale
        rng.standard_normal(50000).astype(np.float32) * np.float32(1e3),
        (rng.random(50000).astype(np.float32) - 0.5) * np.float32(1e-20),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -1.17549435e-38 * 2 ** 20], np.float32),
    ])
    w1, w2, w3 = split3(w)
    assert is_bf16(w1).all() and is_bf16(w2).all() and is_bf16(w3).all()
    # w1 + w2 + w3 in that order, in fp32, gives w back exactly
    assert np.array_equal((w1 + w2 + w3).astype(np.float32).view(np.uint32) & 0x7FFFFFFF,
                          w.view(np.uint32) & 0x7FFFFFFF)
    # and the exact real sum equals w
    assert np.array_equal(w1.astype(np.float64) + w2.astype(np.float64) + w3.astype(np.float64),
                          w.astype(np.float64))


def test_bf16_products_exact_in_fp32():
    rng = np.random.default_rng(1)
    x = bf16_rne(rng.standard_normal(100000).astype(np.float32))
    w1, w2, w3 = split3(rng.standard_normal(100000).astype(np.float32) / np.float32(64))
    for part in (w1, w2, w3):
        p32 = (x * part).astype(np.float32)
        assert np.array_equal(p32.astype(np.float64), x.astype(np.float64) * part.astype(np.float64))
