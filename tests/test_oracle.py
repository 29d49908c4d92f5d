"""Pins for the fp64 oracle: facts the mathematics fixes, independent of the oracle's code.

Each pin is a function of an attention callable ``attn(q, k, v, causal, scale) -> (O, L)``
so that the same pins also run against deliberately broken copies of the
oracle (``test_every_planted_mistake_is_caught``): every plausible slip - a
dropped scale, a transposed product, a flipped or shifted mask, a missing
normalisation, the wrong logarithm - must fail at least one pin.

What pins what:
  * O against ``torch.nn.functional.scaled_dot_product_attention`` in fp64
    (an independent library routine with the same top-left causal mask);
  * L against ``scipy.special.logsumexp`` of the masked logits built with
    ``np.einsum`` (a different routine from the oracle's matmul);
  * closed forms: identical keys, causal row 0, zero queries or zero scale,
    constant V, V = identity (which exposes the softmax matrix itself);
  * pure-Python brute force (math.exp / math.fsum loops) on tiny inputs;
  * invariants: sum_j exp(S_ij - L_i) = 1 (the property that makes L the only
    stored statistic: page "flash-attention123和ring-attention", 优化1),
    permutation equivariance, linearity in V, no overflow at |logit| ~ 1000.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import attention_fp64, attention_rows_fp64

RNG = np.random.default_rng(1234)


def _rand(shape, sigma=1.0, seed=0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


def _masked_logits_einsum(q, k, causal, scale):
    S = scale * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        N = q.shape[2]
        S = np.where(np.triu(np.ones((N, N), dtype=bool), 1), -np.inf, S)
    return S


# --------------------------------------------------------------------------- pins

def pin_sdpa(attn):
    for (B, H, N, d), causal, seed in [((2, 3, 37, 8), False, 1), ((2, 3, 37, 8), True, 2),
                                       ((1, 2, 130, 64), True, 3), ((1, 1, 5, 3), False, 4)]:
        q, k, v = (_rand((B, H, N, d), seed=seed + 10 * t) for t in range(3))
        scale = 0.37 + 0.1 * seed
        O, _ = attn(q, k, v, causal, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=scale).numpy()
        np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def pin_logsumexp(attn):
    for causal, seed in [(False, 5), (True, 6)]:
        q, k, v = (_rand((2, 2, 41, 16), seed=seed + 10 * t) for t in range(3))
        scale = 0.25
        _, L = attn(q, k, v, causal, scale)
        ref = logsumexp(_masked_logits_einsum(q, k, causal, scale), axis=-1)
        np.testing.assert_allclose(L, ref, rtol=0, atol=1e-12)


def pin_identical_keys(attn):
    # K[j] = kvec for every j: every allowed key gets the same weight, so O_i is the
    # mean of the allowed V rows and L_i = scale * q_i . kvec + ln(n_i).
    B, H, N, d = 1, 2, 23, 6
    q = _rand((B, H, N, d), seed=7)
    kvec = _rand((d,), seed=8)
    k = np.broadcast_to(kvec, (B, H, N, d)).copy()
    v = _rand((B, H, N, d), seed=9)
    scale = 0.6
    for causal in (False, True):
        O, L = attn(q, k, v, causal, scale)
        for i in range(N):
            n = i + 1 if causal else N
            np.testing.assert_allclose(O[:, :, i], v[:, :, :n].mean(axis=2), atol=1e-12)
            np.testing.assert_allclose(L[:, :, i], scale * (q[:, :, i] @ kvec) + math.log(n),
                                       atol=1e-12)


def pin_causal_row0(attn):
    q, k, v = (_rand((2, 2, 19, 5), seed=20 + t) for t in range(3))
    scale = 0.9
    O, L = attn(q, k, v, True, scale)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], atol=1e-12)
    np.testing.assert_allclose(L[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1),
                               atol=1e-12)


def pin_zero_logits(attn):
    # Q = 0 (or scale = 0): uniform weights; O is the prefix mean (causal) or the
    # global mean of V, and L_i = ln(i + 1) or ln(N).
    B, H, N, d = 1, 1, 17, 4
    k, v = _rand((B, H, N, d), seed=30), _rand((B, H, N, d), seed=31)
    for q, scale in [(np.zeros((B, H, N, d)), 0.5), (_rand((B, H, N, d), seed=32), 0.0)]:
        for causal in (False, True):
            O, L = attn(q, k, v, causal, scale)
            for i in range(N):
                n = i + 1 if causal else N
                np.testing.assert_allclose(O[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-12)
                np.testing.assert_allclose(L[0, 0, i], math.log(n), atol=1e-12)


def pin_constant_v(attn):
    q, k = _rand((1, 2, 29, 7), seed=40), _rand((1, 2, 29, 7), seed=41)
    v = np.full((1, 2, 29, 7), -2.75)
    for causal in (False, True):
        O, _ = attn(q, k, v, causal, 0.8)
        np.testing.assert_allclose(O, v, atol=1e-12)


def pin_identity_v(attn):
    # V = I (N <= d): row i of O is row i of the softmax matrix itself.
    N, d = 9, 12
    q, k = _rand((1, 1, N, d), seed=50), _rand((1, 1, N, d), seed=51)
    v = np.zeros((1, 1, N, d))
    v[0, 0, :, :N] = np.eye(N)
    for causal in (False, True):
        O, _ = attn(q, k, v, causal, 0.7)
        P = softmax(_masked_logits_einsum(q, k, causal, 0.7), axis=-1)
        np.testing.assert_allclose(O[0, 0, :, :N], P[0, 0], atol=1e-13)
        np.testing.assert_allclose(O[0, 0, :, N:], 0.0, atol=0)


def _brute_python(q, k, v, causal, scale):
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = range(i + 1) if causal else range(N)
                s = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d))
                     for j in js]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                for t in range(d):
                    O[b, h, i, t] = math.fsum(wj * float(v[b, h, j, t]) for wj, j in zip(w, js)) / tot
                L[b, h, i] = mx + math.log(tot)
    return O, L


def pin_brute_force(attn):
    for (B, H, N, d), causal, seed in [((1, 1, 1, 1), False, 60), ((1, 2, 4, 3), True, 61),
                                       ((2, 1, 6, 2), False, 62), ((1, 1, 7, 4), True, 63)]:
        q, k, v = (_rand((B, H, N, d), seed=seed + 100 * t) for t in range(3))
        O, L = attn(q, k, v, causal, 0.45)
        Ob, Lb = _brute_python(q, k, v, causal, 0.45)
        np.testing.assert_allclose(O, Ob, atol=1e-13)
        np.testing.assert_allclose(L, Lb, atol=1e-13)


def pin_weights_sum_to_one(attn):
    q, k, v = (_rand((1, 2, 33, 8), seed=70 + t) for t in range(3))
    for causal in (False, True):
        _, L = attn(q, k, v, causal, 0.5)
        S = _masked_logits_einsum(q, k, causal, 0.5)
        np.testing.assert_allclose(np.exp(S - L[..., None]).sum(axis=-1), 1.0, atol=1e-12)


def pin_large_logits(attn):
    # Logits near +-1000 overflow exp() unless the row max is subtracted first.
    q, k, v = (_rand((1, 1, 24, 4), sigma=s, seed=80 + t) for t, s in enumerate((30.0, 30.0, 1.0)))
    for causal in (False, True):
        O, L = attn(q, k, v, causal, 1.0)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
        ref = logsumexp(_masked_logits_einsum(q, k, causal, 1.0), axis=-1)
        np.testing.assert_allclose(L, ref, rtol=1e-14, atol=1e-9)
        assert np.max(np.abs(L)) > 200.0


def pin_symmetries(attn):
    q, k, v = (_rand((1, 1, 15, 6), seed=90 + t) for t in range(3))
    perm = np.random.default_rng(95).permutation(15)
    O, L = attn(q, k, v, False, 0.5)
    Op, Lp = attn(q, k[:, :, perm], v[:, :, perm], False, 0.5)
    np.testing.assert_allclose(Op, O, atol=1e-13)
    np.testing.assert_allclose(Lp, L, atol=1e-13)
    v2 = _rand((1, 1, 15, 6), seed=96)
    for causal in (False, True):
        Oa, _ = attn(q, k, v, causal, 0.5)
        Ob, _ = attn(q, k, v2, causal, 0.5)
        Oc, _ = attn(q, k, v + 2.0 * v2, causal, 0.5)
        np.testing.assert_allclose(Oc, Oa + 2.0 * Ob, atol=1e-12)


PINS = [pin_sdpa, pin_logsumexp, pin_identical_keys, pin_causal_row0, pin_zero_logits,
        pin_constant_v, pin_identity_v, pin_brute_force, pin_weights_sum_to_one,
        pin_large_logits, pin_symmetries]


def _oracle(q, k, v, causal, scale):
    return attention_fp64(q, k, v, causal=causal, scale=scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_oracle)


# ------------------------------------------------------ planted mistakes, CPU only

def _mutant(kind):
    """A copy of the oracle's definition with one plausible mistake planted in it."""

    def attn(q, k, v, causal, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, d = q.shape
        O = np.zeros((B, H, N, d))
        L = np.zeros((B, H, N))
        for b in range(B):
            for h in range(H):
                s = scale if kind != "no_scale" else 1.0
                S = s * (q[b, h] @ k[b, h].T)
                if kind == "transposed":
                    S = S.T
                if causal:
                    i, j = np.indices((N, N))
                    bad = {"mask_flipped": j < i, "mask_diag": j >= i}.get(kind, j > i)
                    S = np.where(bad, -np.inf, S)
                m = S.max(axis=1)
                if kind == "no_max":
                    m = np.zeros_like(m)
                P = np.exp(S - m[:, None])
                l = P.sum(axis=1)
                if kind == "no_max":
                    m = np.zeros_like(m)
                vv = k[b, h] if kind == "pv_uses_k" else v[b, h]
                O[b, h] = (P @ vv) if kind == "no_norm" else (P @ vv) / l[:, None]
                if kind == "log2":
                    L[b, h] = m + np.log2(l)
                elif kind == "dropped_m":
                    L[b, h] = np.log(l)
                elif kind == "unscaled_L":
                    L[b, h] = (m / s if s else m) + np.log(l)
                else:
                    L[b, h] = m + np.log(l)
        return O, L

    return attn


MUTANTS = ["no_scale", "transposed", "mask_flipped", "mask_diag", "no_max", "pv_uses_k",
           "no_norm", "log2", "dropped_m", "unscaled_L"]


def test_unmutated_copy_passes_every_pin():
    # The mutation harness itself, with no mistake planted, must pass every pin.
    for pin in PINS:
        pin(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_planted_mistake_is_caught(kind):
    attn = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {kind!r} slipped past every pin"


# ------------------------------------------------------------ row sampler

def test_rows_sampler_matches_full_oracle():
    q, k, v = (_rand((2, 3, 70, 8), seed=110 + t) for t in range(3))
    for causal in (False, True):
        O, L = attention_fp64(q, k, v, causal=causal, scale=0.3)
        rows = [0, 1, 33, 69]
        Or, Lr = attention_rows_fp64(q, k, v, 1, 2, rows, causal=causal, scale=0.3)
        np.testing.assert_array_equal(Or, O[1, 2, rows])
        np.testing.assert_array_equal(Lr, L[1, 2, rows])


def test_row_chunking_does_not_change_result():
    q, k, v = (_rand((1, 1, 50, 4), seed=120 + t) for t in range(3))
    for causal in (False, True):
        O1, L1 = attention_fp64(q, k, v, causal=causal, scale=0.5, row_chunk=7)
        O2, L2 = attention_fp64(q, k, v, causal=causal, scale=0.5, row_chunk=4096)
        np.testing.assert_allclose(O1, O2, atol=1e-14)
        np.testing.assert_allclose(L1, L2, atol=1e-14)


def test_bf16_inputs_upcast_exactly():
    # The oracle must see exactly the bf16 bits the GPU sees: torch bf16 -> fp64 is exact.
    q = torch.randn(1, 1, 8, 4).to(torch.bfloat16)
    O, L = attention_fp64(q, q, q, causal=True)
    qf = q.to(torch.float64).numpy()
    O2, L2 = attention_fp64(qf, qf, qf, causal=True)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = (_rand((1, 1, 6, 16), seed=130 + t) for t in range(3))
    O1, L1 = attention_fp64(q, k, v)
    O2, L2 = attention_fp64(q, k, v, scale=0.25)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)
