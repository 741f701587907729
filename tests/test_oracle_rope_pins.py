"""Pins of the RoPE oracle against things other than itself: the complex
exponential form with frequencies written out as numbers, the
relative-position property, the identity at position 0, and the pages'
statement that absolute positions make chunked prefill equal to one
monolithic pass.  Each planted mistake at the end must break one of them.
CPU only."""
import math

import numpy as np
import pytest

from oracle import attention as oa
from oracle import rope as orope
from tests.oracle_helpers import empty_pools, run_chunked

# theta = 10000, D = 8: the four pairs turn by 1, 1e-1, 1e-2, 1e-3 rad per
# position (theta ** (-2i/D) for i = 0..3, evaluated by hand)
FREQ_D8 = np.array([1.0, 0.1, 0.01, 0.001])


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _complex_view(x, interleaved):
    d = x.shape[-1]
    if interleaved:
        return x[..., 0::2] + 1j * x[..., 1::2]
    return x[..., : d // 2] + 1j * x[..., d // 2:]


@pytest.mark.parametrize("interleaved", [False, True])
def test_pairs_turn_as_complex_exponentials(interleaved):
    x = _rand(1, 5, 3, 8)
    pos = np.array([0, 1, 7, 100, 32767])
    got = _complex_view(orope.rotate(x, pos, 10000.0, interleaved), interleaved)
    ref = _complex_view(x, interleaved) * np.exp(1j * pos[:, None, None] * FREQ_D8[None, None, :])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_frequencies_are_the_printed_numbers():
    np.testing.assert_allclose(orope.inv_freq(8, 10000.0), FREQ_D8, rtol=1e-15, atol=0)
    np.testing.assert_allclose(orope.inv_freq(4, 10000.0), [1.0, 0.01], rtol=1e-15, atol=0)


def test_unit_vector_turns_counterclockwise():
    # e_0 at position 1 with D = 2: (1, 0) -> (cos 1, sin 1)
    x = np.array([[[1.0, 0.0]]])
    got = orope.rotate(x, [1], 10000.0)
    np.testing.assert_allclose(got[0, 0], [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)


@pytest.mark.parametrize("interleaved", [False, True])
def test_scores_depend_only_on_relative_position(interleaved):
    q, k = _rand(2, 1, 1, 16), _rand(3, 1, 1, 16)
    for p, s, shift in [(5, 2, 100), (0, 0, 12345), (3000, 17, 7), (9, 40, 1)]:
        a = np.sum(orope.rotate(q, [p], 10000.0, interleaved) * orope.rotate(k, [s], 10000.0, interleaved))
        b = np.sum(orope.rotate(q, [p + shift], 10000.0, interleaved)
                   * orope.rotate(k, [s + shift], 10000.0, interleaved))
        c = np.sum(q * orope.rotate(k, [s - p], 10000.0, interleaved))
        assert abs(a - b) < 1e-11 and abs(a - c) < 1e-11


def test_position_zero_is_identity_and_norms_are_kept():
    x = _rand(4, 6, 2, 16)
    np.testing.assert_array_equal(orope.rotate(x, np.zeros(6, dtype=int), 500000.0), x)
    y = orope.rotate(x, np.arange(6) * 1000, 500000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)


def test_token_positions_follow_cached_lengths():
    pos = orope.token_positions([0, 3, 3, 7], [10, 4, 0])
    np.testing.assert_array_equal(pos, [10, 11, 12, 0, 1, 2, 3])


def _rope_prompt(q, k, v, chunks, block_size, table, num_blocks, num_kv_heads, scale, theta):
    """Chunk by chunk: rotate at absolute positions, write, attend."""
    k_pool, v_pool = empty_pools(num_blocks, block_size, num_kv_heads, q.shape[2])
    outs, c = [], 0
    for n in chunks:
        cu, cached = [0, n], [c]
        qr, k_pool, v_pool = orope.rope_cache_write(q[c:c + n], k_pool, v_pool, k[c:c + n],
                                                    v[c:c + n], [table], cu, cached, block_size,
                                                    theta)
        outs.append(oa.attention(qr, k_pool, v_pool, [table], cu, cached, block_size, scale,
                                 num_kv_heads))
        c += n
    return np.concatenate(outs)


def test_chunked_equals_monolithic_with_rope():
    H, G, D, bs, P = 4, 2, 16, 8, 90
    q, k, v = _rand(5, P, H, D), _rand(6, P, G, D), _rand(7, P, G, D)
    table = np.random.default_rng(8).permutation(16)[:12]
    scale = 1 / math.sqrt(D)
    mono = _rope_prompt(q, k, v, [P], bs, table, 16, G, scale, 100.0)
    chunked = _rope_prompt(q, k, v, [32, 32, 17, 9], bs, table, 16, G, scale, 100.0)
    np.testing.assert_allclose(chunked, mono, rtol=0, atol=1e-12)
    # and RoPE is not the identity on this prompt
    plain, _, _ = run_chunked(q, k, v, [P], bs, table, 16, G, scale)
    assert np.abs(plain - mono).max() > 1e-2


# --------------------------------------------------------------------------
# Planted mistakes (in the oracle, on the CPU): each must fail some pin.
# --------------------------------------------------------------------------
def _relative_positions(cu_seqlens_q, cached_seq_len):
    total = int(cu_seqlens_q[-1])
    pos = np.empty(total, dtype=np.int64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        pos[q0:q1] = np.arange(q1 - q0)
    return pos


def _freq_missing_two(head_dim, theta):
    return np.power(float(theta), -np.arange(head_dim // 2, dtype=np.float64) / head_dim)


def _rotate_one_sign_flipped(x, positions, theta, interleaved=False):
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(positions, dtype=np.float64)[:, None] * orope.inv_freq(x.shape[-1], theta)[None, :]
    cos, sin = np.cos(a)[:, None, :], np.sin(a)[:, None, :]
    i0, i1 = orope.pair_index(x.shape[-1], interleaved)
    out = np.empty_like(x)
    out[..., i0] = x[..., i0] * cos - x[..., i1] * sin
    out[..., i1] = -x[..., i0] * sin + x[..., i1] * cos
    return out


def _halves_paired_as_neighbours(head_dim, interleaved):
    i = np.arange(head_dim // 2)
    return 2 * i, 2 * i + 1


PINS = [
    lambda: test_pairs_turn_as_complex_exponentials(False),
    lambda: test_pairs_turn_as_complex_exponentials(True),
    test_frequencies_are_the_printed_numbers,
    test_unit_vector_turns_counterclockwise,
    lambda: test_scores_depend_only_on_relative_position(False),
    test_position_zero_is_identity_and_norms_are_kept,
    test_token_positions_follow_cached_lengths,
    test_chunked_equals_monolithic_with_rope,
]


@pytest.mark.parametrize("name,attr,bad", [
    ("chunk-relative positions", "token_positions", _relative_positions),
    ("exponent without the factor 2", "inv_freq", _freq_missing_two),
    ("one rotation sign flipped", "rotate", _rotate_one_sign_flipped),
    ("rotate-half pairs taken as neighbours", "pair_index", _halves_paired_as_neighbours),
])
def test_planted_rope_mistake_is_caught(monkeypatch, name, attr, bad):
    monkeypatch.setattr(orope, attr, bad)
    failures = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1, f"no pin caught: {name}"
