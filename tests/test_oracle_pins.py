"""The CPU oracle against hand-worked values, closed forms, exact arithmetic
and brute force (see tests/pins.py), plus round trips of the canonical words."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import qref
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(qref)


@settings(max_examples=60, deadline=None)
@given(fmt=st.sampled_from([0, 1, 2, 3]), n=st.integers(1, 5), kw=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1))
def test_word_roundtrip(fmt, n, kw, seed):
    rng = np.random.default_rng(seed)
    cpw = 32 // oracle.BITS[fmt]
    words = rng.integers(0, 2**32, size=(n, kw), dtype=np.uint64).astype(np.uint32)
    codes = oracle.unpack_codes(words, n, kw * cpw, fmt)
    assert codes.max(initial=0) < (1 << oracle.BITS[fmt])
    assert np.array_equal(oracle.pack_codes(codes, fmt), words)
    assert np.array_equal(pins.pack_literal(codes, oracle.BITS[fmt]), words)


@settings(max_examples=40, deadline=None)
@given(fmt=st.sampled_from([0, 1, 2, 3]), n=st.integers(1, 4), kw=st.integers(1, 4),
       seed=st.integers(0, 2**31 - 1))
def test_code_roundtrip(fmt, n, kw, seed):
    rng = np.random.default_rng(seed)
    b = oracle.BITS[fmt]
    K = kw * (32 // b)
    codes = rng.integers(0, 1 << b, size=(n, K), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(codes, fmt), n, K, fmt), codes)


def test_empty_output():
    y = oracle.qgemm_ref(np.zeros((0, 64), np.float16), np.zeros((4, 8), np.uint32),
                         np.ones((4, 2), np.float16), np.zeros((4, 2), np.float16), 0, 4, 64, 32, 0)
    assert y.shape == (0, 4)
