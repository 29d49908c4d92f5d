"""Pins for the oracle when the query and key lengths differ (Nq != Nk).

The grid on the pages is sized by the query length alone (page "FlashAttention学习笔记(2)",
section "V2中的thread blocks排布"), so Q may have a different length from K and V.  The causal
mask is then aligned bottom-right (key j hidden from row i when j > i + Nk - Nq): the last query
sees every key, as in decoding or in a prompt appended to a cache.

What pins what:
  * non-causal O against ``torch.nn.functional.scaled_dot_product_attention`` in fp64 and L
    against ``scipy.special.logsumexp`` (library routines, any lengths);
  * Nq < Nk, causal: the result is the last Nq rows of the square causal problem whose queries
    end with these Nq rows (the square problem is pinned on its own in test_oracle.py);
  * Nq > Nk, causal: the first Nq - Nk rows see no key (O = 0, L = -inf); the others are the
    square causal problem of the last Nk queries;
  * a single query sees every key under either mask;
  * no keys at all: O = 0, L = -inf;
  * pure-Python brute force on tiny inputs;
  * planted mistakes (top-left alignment, the offset with the wrong sign, NaN for rows that
    see nothing) must each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention_fp64, attention_rows_fp64


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(B, H, Nq, Nk, d, seed):
    return _rand((B, H, Nq, d), seed), _rand((B, H, Nk, d), seed + 1), _rand((B, H, Nk, d), seed + 2)


# --------------------------------------------------------------------------- pins

def pin_noncausal_library(attn):
    for Nq, Nk, seed in [(1, 40, 1), (7, 3, 2), (50, 129, 3), (64, 17, 4)]:
        q, k, v = _qkv(2, 2, Nq, Nk, 8, seed)
        O, L = attn(q, k, v, False, 0.41)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.41).numpy()
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
        Lref = logsumexp(0.41 * np.einsum("bhid,bhjd->bhij", q, k), axis=-1)
        np.testing.assert_allclose(L, Lref, rtol=0, atol=1e-12)


def pin_short_queries_are_the_last_rows_of_the_square_problem(attn):
    for Nq, Nk, seed in [(1, 9, 5), (5, 33, 6), (31, 32, 7), (40, 130, 8)]:
        qfull, k, v = _qkv(1, 2, Nk, Nk, 6, seed)
        q = qfull[:, :, Nk - Nq:].copy()
        O, L = attn(q, k, v, True, 0.5)
        Of, Lf = attn(qfull, k, v, True, 0.5)
        np.testing.assert_allclose(O, Of[:, :, Nk - Nq:], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, Lf[:, :, Nk - Nq:], rtol=0, atol=1e-13)


def pin_excess_queries_see_nothing_then_the_square_problem(attn):
    for Nq, Nk, seed in [(9, 1, 9), (33, 5, 10), (130, 40, 11)]:
        q, k, v = _qkv(1, 2, Nq, Nk, 6, seed)
        O, L = attn(q, k, v, True, 0.5)
        e = Nq - Nk
        assert np.all(O[:, :, :e] == 0.0) and np.all(L[:, :, :e] == -np.inf)
        Os, Ls = attn(q[:, :, e:].copy(), k, v, True, 0.5)
        np.testing.assert_allclose(O[:, :, e:], Os, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, :, e:], Ls, rtol=0, atol=1e-13)


def pin_single_query_sees_every_key(attn):
    q, k, v = _qkv(2, 3, 1, 77, 16, 12)
    Oc, Lc = attn(q, k, v, True, 0.3)
    On, Ln = attn(q, k, v, False, 0.3)
    np.testing.assert_allclose(Oc, On, rtol=0, atol=0)
    np.testing.assert_allclose(Lc, Ln, rtol=0, atol=0)
    w = np.exp(0.3 * np.einsum("bhd,bhjd->bhj", q[:, :, 0], k))
    np.testing.assert_allclose(Oc[:, :, 0], np.einsum("bhj,bhjd->bhd", w, v) / w.sum(-1)[..., None],
                               rtol=0, atol=1e-12)


def pin_no_keys(attn):
    q = _rand((1, 2, 5, 4), 13)
    k = np.zeros((1, 2, 0, 4))
    for causal in (False, True):
        O, L = attn(q, k, k.copy(), causal, 1.0)
        assert O.shape == (1, 2, 5, 4) and np.all(O == 0.0) and np.all(L == -np.inf)


def _brute_python(q, k, v, causal, scale):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, Nq, d))
    L = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if not (causal and j - i > Nk - Nq)]
                if not keys:
                    continue
                s = {j: scale * math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) for j in keys}
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                tot = math.fsum(w.values())
                for t in range(d):
                    O[b, h, i, t] = math.fsum(w[j] * v[b, h, j, t] for j in keys) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def pin_brute_force(attn):
    for Nq, Nk, causal, seed in [(3, 5, True, 14), (5, 3, True, 15), (4, 6, False, 16), (6, 2, True, 17)]:
        q, k, v = _qkv(1, 2, Nq, Nk, 3, seed)
        O, L = attn(q, k, v, causal, 0.8)
        Ob, Lb = _brute_python(q, k, v, causal, 0.8)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


PINS = [pin_noncausal_library, pin_short_queries_are_the_last_rows_of_the_square_problem,
        pin_excess_queries_see_nothing_then_the_square_problem, pin_single_query_sees_every_key,
        pin_no_keys, pin_brute_force]


def _oracle(q, k, v, causal, scale):
    return attention_fp64(q, k, v, causal=causal, scale=scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_oracle)


# ---------------------------------------------------------------- planted mistakes

def _mutant(kind):
    """A copy of the definition with one plausible slip."""

    def attn(q, k, v, causal, scale):
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        off = {"topleft": 0, "flipped": Nq - Nk}.get(kind, Nk - Nq)
        O = np.zeros((B, H, Nq, d))
        L = np.full((B, H, Nq), -np.inf)
        if Nk == 0:
            return O, L
        S = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            S = np.where(np.arange(Nk)[None, :] > np.arange(Nq)[:, None] + off, -np.inf, S)
        with np.errstate(invalid="ignore"):
            m = S.max(-1, keepdims=True)
            P = np.exp(S - m)
            l = P.sum(-1, keepdims=True)
            O = P @ v / l
            L = (m + np.log(l))[..., 0]
        if kind != "nan_rows":
            seen = np.isfinite(m[..., 0])
            O = np.where(seen[..., None], O, 0.0)
            L = np.where(seen, L, -np.inf)
        return O, L

    return attn


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", ["topleft", "flipped", "nan_rows"])
def test_every_planted_mistake_is_caught(kind):
    failed = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {kind!r} passed every pin"


def test_rows_sampler_matches_full_oracle_for_both_length_orders():
    for Nq, Nk in [(20, 70), (70, 20)]:
        q, k, v = _qkv(2, 2, Nq, Nk, 8, 18)
        O, L = attention_fp64(q, k, v, causal=True, scale=0.4)
        rows = [0, 3, Nq // 2, Nq - 1]
        Or, Lr = attention_rows_fp64(q, k, v, 1, 0, rows, causal=True, scale=0.4)
        # the same rows through a smaller matmul: equal up to the BLAS's summation order
        np.testing.assert_allclose(Or, O[1, 0, rows], rtol=0, atol=1e-14)
        np.testing.assert_allclose(Lr, L[1, 0, rows], rtol=0, atol=1e-14)


def test_fp16_inputs_upcast_exactly():
    x = torch.randn(2, 3, 5, 8).to(torch.float16)
    O, L = attention_fp64(x, x, x, causal=True)
    O2, L2 = attention_fp64(x.double().numpy(), x.double().numpy(), x.double().numpy(), causal=True)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
