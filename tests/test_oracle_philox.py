"""Pins of the oracle's Philox4x64-10 uniforms against numpy's own Philox bit generator
(numpy.random.Philox, the same published algorithm), driven with an explicit key and counter:
its raw 64-bit words for counter c come from the block at c + 1 (it advances the counter
before each block)."""

import numpy as np
import pytest

import oracle.spec_verify_oracle as O


@pytest.mark.parametrize("key,counter", [((0, 0), 0), ((5, 7), 0), ((2**64 - 1, 3), 2**64 - 3),
                                          ((123456789, 987654321), 2**130 + 17)])
def test_blocks_match_numpy(key, counter):
    ctr_words = np.array([(counter >> (64 * j)) & (2**64 - 1) for j in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=ctr_words)
    raw = bg.random_raw(12)
    for blk in range(3):
        c = counter + 1 + blk
        words = O.philox4x64([(c >> (64 * j)) & (2**64 - 1) for j in range(4)], key)
        assert [int(v) for v in raw[4 * blk: 4 * blk + 4]] == words


def test_uniform_mapping_and_stream_layout():
    key, counter = (11, 22), 40
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array([counter - 1, 0, 0, 0], dtype=np.uint64))
    raw = bg.random_raw(10)
    u = O.philox_uniforms(key, counter, 10)
    expect = ((raw >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
    np.testing.assert_array_equal(u, expect)
    assert u.dtype == np.float32 and (u >= 0).all() and (u < 1).all()
    # a later start continues the same stream
    np.testing.assert_array_equal(O.philox_uniforms(key, counter + 1, 6), u[4:10])


def test_uniform_statistics():
    u = O.philox_uniforms((3, 4), 0, 40000).astype(np.float64)
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005
    hist = np.histogram(u, bins=10, range=(0, 1))[0]
    chi2 = float(np.sum((hist - 4000) ** 2 / 4000))
    assert chi2 < 21.67  # df = 9, 1%


def test_planted_mistake_fails():
    """Rounds dropped (9 instead of 10) no longer match numpy."""
    bg = np.random.Philox(key=np.array([1, 2], dtype=np.uint64),
                          counter=np.zeros(4, dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(4)]
    assert O.philox4x64([1, 0, 0, 0], (1, 2), rounds=9) != raw
    assert O.philox4x64([1, 0, 0, 0], (1, 2)) == raw
