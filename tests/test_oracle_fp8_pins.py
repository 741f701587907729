"""Pins of the FP8 (E4M3) oracle: torch's float8_e4m3fn conversion (a
library routine) for every code and for random in-range values, values
worked out by hand (largest, smallest, ties, saturation), round trips, and
planted mistakes.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import fp8 as of8


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = of8.decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_encode_matches_torch_on_random_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of8.encode(x.astype(np.float64)), ref)


def test_hand_values():
    cases = {448.0: 0x7E, 1.0: 0x38, 2.0 ** -9: 0x01, -2.0: 0xC0, 0.0: 0x00, 2.0 ** -6: 0x08,
             -1e-4: 0x80,       # rounds to zero, keeps its sign
             1.0625: 0x38,      # halfway 1 .. 1.125: even code 1.0
             1.1875: 0x3A,      # halfway 1.125 .. 1.25: even code 1.25
             432.0: 0x7E,       # halfway 416 .. 448: even code (0x7E) 448
             500.0: 0x7E, -1e6: 0xFE}   # saturation
    for x, code in cases.items():
        assert int(of8.encode(np.array([x]))[0]) == code, (x, hex(code))
    assert of8.MAX == 448.0


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(of8.encode(of8.decode(codes)), codes)


def test_quantize_scales_in_float32():
    x = np.array([0.3, -7.0, 1000.0], dtype=np.float32)
    codes = of8.quantize(x, 0.5)
    assert np.array_equal(of8.decode(codes), [0.625, -14.0, 448.0])


# planted mistakes
def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), of8.MAX)
    idx = np.argmin(np.abs(of8.GRID[None, :] - a[:, None]) - 1e-12 * of8.GRID[None, :], axis=1)
    code = idx.astype(np.uint8)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _grid_wrong_bias():
    return np.array([m / 8.0 * 2.0 ** -7 if (c >> 3) == 0 else (1 + m / 8.0) * 2.0 ** ((c >> 3) - 8)
                     for c in range(0x7F) for m in [c & 7]])


PINS = [test_decode_matches_torch_for_every_code, test_encode_matches_torch_on_random_values,
        test_hand_values, test_every_finite_code_round_trips]


@pytest.mark.parametrize("name", ["ties away from zero", "exponent bias 8"])
def test_planted_fp8_mistake_is_caught(monkeypatch, name):
    if name == "ties away from zero":
        monkeypatch.setattr(of8, "encode", _encode_ties_away)
    else:
        monkeypatch.setattr(of8, "GRID", _grid_wrong_bias())
    failures = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught: {name}"


def test_fp8_cache_chunked_equals_monolithic():
    # quantization is per element and position-free: the attention over a
    # chunked fp8 cache equals the one over the whole prompt written at once
    import math
    from oracle import attention as oa
    H, G, D, bs, P = 4, 2, 16, 8, 70
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal(s) for s in ((P, H, D), (P, G, D), (P, G, D)))
    table = rng.permutation(12)[:9]
    pool = np.zeros((12, bs, G, D), dtype=np.uint8)

    def run(chunks):
        kp, vp, outs, c = pool, pool, [], 0
        for n in chunks:
            kp, vp = of8.cache_write(kp, vp, k[c:c + n], v[c:c + n], [table], [0, n], [c], bs, 0.5, 2.0)
            outs.append(oa.attention(q[c:c + n], of8.dequantize(kp, 0.5), of8.dequantize(vp, 2.0),
                                     [table], [0, n], [c], bs, 1 / math.sqrt(D), G))
            c += n
        return np.concatenate(outs)

    np.testing.assert_allclose(run([30, 30, 10]), run([P]), rtol=0, atol=1e-12)
