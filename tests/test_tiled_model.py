"""The tiled FlashAttention-2 algorithm (fp64 CPU model) against the plain definition.

These pin the identities the pages state and the GPU kernel relies on:
  * the Q-outer / KV-inner loop with a running max and sum reaches the global
    softmax result once every K/V block has been visited (page
    "Flash Attention V2原理解读", commentary on the FWD inner loop) - checked by
    brute force over many tile shapes, ragged lengths and Br != Bc;
  * normalising once at the end equals normalising every step (page
    "flash-attention123和ring-attention", 优化2);
  * skipping K/V blocks that the causal mask covers entirely changes nothing
    (same page, 优化3) - bit for bit, since such blocks only add exact zeros;
  * the number of blocks each causal query block visits.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import attention_fp64, causal_block_end, fa2_forward_tiled_fp64


def _rand(shape, seed, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_definition_bruteforce(causal):
    seed = 0
    for N in list(range(1, 21)) + [31, 40]:
        for d in (1, 3, 16):
            q, k, v = (_rand((1, 1, N, d), seed + t) for t in range(3))
            seed += 3
            O, L = attention_fp64(q, k, v, causal=causal, scale=0.6)
            for Br, Bc in itertools.product((1, 2, 3, 5, 8, 16), (1, 3, 4, 7, 16, 64)):
                Ot, Lt = fa2_forward_tiled_fp64(q, k, v, causal=causal, scale=0.6, Br=Br, Bc=Bc)
                np.testing.assert_allclose(Ot, O, rtol=0, atol=1e-12, err_msg=f"N={N} d={d} {Br}x{Bc}")
                np.testing.assert_allclose(Lt, L, rtol=0, atol=1e-12, err_msg=f"N={N} d={d} {Br}x{Bc}")


@settings(max_examples=60, deadline=None)
@given(B=st.integers(1, 2), H=st.integers(1, 2), N=st.integers(1, 70), d=st.integers(1, 12),
       Br=st.integers(1, 40), Bc=st.integers(1, 40), causal=st.booleans(),
       sigma=st.sampled_from([0.1, 1.0, 8.0]), seed=st.integers(0, 2**31 - 1))
def test_tiled_equals_definition_random(B, H, N, d, Br, Bc, causal, sigma, seed):
    q, k, v = (_rand((B, H, N, d), seed + t, sigma if t < 2 else 1.0) for t in range(3))
    O, L = attention_fp64(q, k, v, causal=causal, scale=0.5)
    Ot, Lt = fa2_forward_tiled_fp64(q, k, v, causal=causal, scale=0.5, Br=Br, Bc=Bc)
    np.testing.assert_allclose(Ot, O, rtol=0, atol=1e-11)
    np.testing.assert_allclose(Lt, L, rtol=1e-13, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_deferred_normalisation_equals_per_step(causal):
    for N, Br, Bc, seed in [(37, 8, 5, 1), (64, 16, 16, 2), (100, 32, 7, 3)]:
        q, k, v = (_rand((2, 2, N, 8), seed * 10 + t) for t in range(3))
        Od, Ld = fa2_forward_tiled_fp64(q, k, v, causal=causal, Br=Br, Bc=Bc, deferred_norm=True)
        Os, Ls = fa2_forward_tiled_fp64(q, k, v, causal=causal, Br=Br, Bc=Bc, deferred_norm=False)
        np.testing.assert_allclose(Od, Os, rtol=0, atol=1e-13)
        np.testing.assert_array_equal(Ld, Ls)


def test_causal_block_skip_is_bitwise_neutral():
    for N, Br, Bc, seed in [(37, 8, 5, 1), (64, 16, 16, 2), (100, 32, 7, 3), (130, 64, 32, 4),
                            (9, 2, 9, 5)]:
        q, k, v = (_rand((1, 2, N, 8), seed * 10 + t) for t in range(3))
        Os, Ls = fa2_forward_tiled_fp64(q, k, v, causal=True, Br=Br, Bc=Bc, skip_masked=True)
        Oa, La = fa2_forward_tiled_fp64(q, k, v, causal=True, Br=Br, Bc=Bc, skip_masked=False)
        np.testing.assert_array_equal(Os, Oa)
        np.testing.assert_array_equal(Ls, La)


def test_causal_block_end_counts():
    # Square tiles: query block i visits blocks 0..i.
    assert [causal_block_end(i, 64, 64, 256) for i in range(4)] == [1, 2, 3, 4]
    # Br = 2 Bc: block i needs keys up to (i+1)*Br - 1.
    assert [causal_block_end(i, 128, 64, 512) for i in range(4)] == [2, 4, 6, 8]
    # Ragged last block: only keys up to N - 1 exist.
    assert causal_block_end(1, 128, 64, 200) == 4
    assert causal_block_end(0, 128, 64, 1) == 1
    # Every block that is visited holds at least one key <= the block's last row,
    # and the first block not visited holds none.
    for N, Br, Bc in [(100, 16, 7), (8191, 128, 64), (257, 64, 128)]:
        for i in range(-(-N // Br)):
            e = causal_block_end(i, Br, Bc, N)
            last = min(N, (i + 1) * Br) - 1
            assert (e - 1) * Bc <= last < e * Bc


def test_logits_near_100_stay_finite():
    # The ragged stress workload draws Q, K with sigma 4, d = 256: scaled logits reach ~100,
    # past fp32's exp overflow at 88.7.  The running max keeps every exp <= 1.
    q, k = _rand((1, 1, 64, 256), 1, 4.0), _rand((1, 1, 64, 256), 2, 4.0)
    v = np.random.default_rng(3).uniform(-1, 1, (1, 1, 64, 256))
    O, L = attention_fp64(q, k, v, causal=True)
    Ot, Lt = fa2_forward_tiled_fp64(q, k, v, causal=True, Br=16, Bc=8)
    assert np.abs(L).max() > 40  # logit std is 16 here
    np.testing.assert_allclose(Ot, O, atol=1e-12)
    np.testing.assert_allclose(Lt, L, rtol=1e-15, atol=1e-11)
