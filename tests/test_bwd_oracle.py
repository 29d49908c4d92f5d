"""Pins for the backward oracle (oracle/backward.py).

What pins what:
  * the gradients against torch.autograd in float64 through an explicit softmax attention (a
    separate, library-differentiated code path), with and without the causal mask;
  * central finite differences of sum(O * dO) on tiny inputs, element by element;
  * closed forms: dO = 0 gives zero gradients; identical V rows give dQ = dK = 0 (every key
    carries the same value, so the scores do not matter) and dV = P^T dO; a single key gives
    dQ = dK = 0 and dV = dO summed over rows;
  * the identity rowsum(dO * O) = rowsum(P * dP) behind the D term;
  * planted mistakes (no D term, dS^T vs dS in dK, a missing scale, the mask on the wrong side)
    must each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle.backward import attention_bwd_fp64, delta_fp64


def _qkv(B, H, N, d, seed, sigma=1.0):
    g = np.random.default_rng(seed)
    q, k = g.standard_normal((2, B, H, N, d)) * sigma
    v, do = g.standard_normal((2, B, H, N, d))
    return q, k, v, do


def _autograd(q, k, v, do, causal, scale):
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    S = scale * torch.matmul(t[0], t[1].transpose(-1, -2))
    if causal:
        N = q.shape[-2]
        S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    O = torch.matmul(torch.softmax(S, dim=-1), t[2])
    O.backward(torch.tensor(do, dtype=torch.float64))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 4), (2, 3, 17, 8), (1, 2, 64, 16)])
def test_against_autograd(shape, causal):
    q, k, v, do = _qkv(*shape, seed=sum(shape) + causal)
    scale = 0.3
    got = attention_bwd_fp64(q, k, v, do, causal, scale)
    ref = _autograd(q, k, v, do, causal, scale)
    for g, r in zip(got, ref):
        assert np.abs(g - r).max() < 1e-12


def test_finite_differences():
    q, k, v, do = _qkv(1, 1, 5, 3, seed=4)
    scale = 0.7

    def loss(q_, k_, v_):
        S = scale * q_[0, 0] @ k_[0, 0].T
        S = np.where(np.arange(5)[None, :] > np.arange(5)[:, None], -np.inf, S)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        return float(((P @ v_[0, 0]) * do[0, 0]).sum())

    dQ, dK, dV = attention_bwd_fp64(q, k, v, do, True, scale)
    eps = 1e-6
    for grad, which in ((dQ, 0), (dK, 1), (dV, 2)):
        for idx in [(0, 0, 0, 0), (0, 0, 2, 1), (0, 0, 4, 2), (0, 0, 3, 0)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            assert abs((up - dn) / (2 * eps) - grad[idx]) < 1e-7


def test_zero_upstream_gradient():
    q, k, v, _ = _qkv(1, 2, 9, 4, seed=5)
    for g in attention_bwd_fp64(q, k, v, np.zeros_like(q), True, 0.5):
        assert np.all(g == 0)


def test_identical_value_rows():
    q, k, _, do = _qkv(1, 1, 11, 4, seed=6)
    v = np.broadcast_to(np.array([0.5, -1.0, 2.0, 3.0]), (1, 1, 11, 4)).copy()
    dQ, dK, dV = attention_bwd_fp64(q, k, v, do, False, 0.4)
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13
    S = 0.4 * q[0, 0] @ k[0, 0].T
    P = np.exp(S - S.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    assert np.abs(dV[0, 0] - P.T @ do[0, 0]).max() < 1e-13


def test_single_key():
    q, k, v, do = _qkv(1, 1, 1, 6, seed=7)
    dQ, dK, dV = attention_bwd_fp64(q, k, v, do, True, 1.3)
    # P = 1, so dS = dP - D = dO.v - dO.v: zero up to the rounding of two dot products
    assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-14
    assert np.abs(dV - do).max() < 1e-15


def test_delta_identity():
    q, k, v, do = _qkv(2, 2, 13, 5, seed=8)
    scale = 0.45
    for causal in (False, True):
        S = scale * np.einsum("bhid,bhjd->bhij", q, k)
        if causal:
            S = np.where(np.arange(13)[None, :] > np.arange(13)[:, None], -np.inf, S)
        P = np.exp(S - S.max(-1, keepdims=True))
        P /= P.sum(-1, keepdims=True)
        O = P @ v
        dP = do @ np.swapaxes(v, -1, -2)
        assert np.abs(delta_fp64(O, do) - (P * dP).sum(-1)).max() < 1e-12


# ---- planted mistakes ------------------------------------------------------------------------
def _broken(kind):
    def f(q, k, v, do, causal, scale):
        dQ, dK, dV = [], [], []
        for b in range(q.shape[0]):
            rq, rk, rv = [], [], []
            for h in range(q.shape[1]):
                S = scale * q[b, h] @ k[b, h].T
                N = S.shape[0]
                if causal:
                    hide = np.arange(N)[None, :] < np.arange(N)[:, None] if kind == "mask" else \
                        np.arange(N)[None, :] > np.arange(N)[:, None]
                    S = np.where(hide, -np.inf, S)
                P = np.exp(S - S.max(1, keepdims=True))
                P /= P.sum(1, keepdims=True)
                dP = do[b, h] @ v[b, h].T
                D = 0.0 if kind == "noD" else (P * dP).sum(1, keepdims=True)
                dS = P * (dP - D)
                rq.append((1.0 if kind == "noscale" else scale) * dS @ k[b, h])
                rk.append(scale * (dS @ q[b, h] if kind == "transpose" else dS.T @ q[b, h]))
                rv.append(P.T @ do[b, h])
            dQ.append(rq), dK.append(rk), dV.append(rv)
        return np.array(dQ), np.array(dK), np.array(dV)
    return f


@pytest.mark.parametrize("kind", ["noD", "transpose", "noscale", "mask"])
def test_every_planted_mistake_is_caught(kind):
    q, k, v, do = _qkv(1, 2, 9, 4, seed=9)
    got = _broken(kind)(q, k, v, do, True, 0.3)
    ref = _autograd(q, k, v, do, True, 0.3)
    assert max(np.abs(g - r).max() for g, r in zip(got, ref)) > 1e-6


# ---- query and key lengths that differ (bottom-right causal alignment) ----------------------
@pytest.mark.parametrize("Nq,Nk", [(3, 11), (11, 3), (1, 9), (16, 16)])
def test_noncausal_lengths_against_autograd(Nq, Nk):
    g = np.random.default_rng(Nq * 31 + Nk)
    q, do = g.standard_normal((2, 2, 2, Nq, 8))
    k, v = g.standard_normal((2, 2, 2, Nk, 8))
    got = attention_bwd_fp64(q, k, v, do, False, 0.35)
    ref = _autograd(q, k, v, do, False, 0.35)
    for a, b in zip(got, ref):
        assert a.shape == b.shape and np.abs(a - b).max() < 1e-12


@pytest.mark.parametrize("Nq,Nk", [(1, 9), (4, 13), (12, 13)])
def test_short_queries_are_the_last_rows_of_the_square_problem(Nq, Nk):
    # The square causal problem with Nk queries, the first Nk - Nq of which have dO = 0:
    # those rows add nothing to dK and dV, and the other rows see exactly the keys the
    # bottom-right mask gives the Nq queries.
    g = np.random.default_rng(Nq + 7 * Nk)
    qf, dof, k, v = g.standard_normal((4, 1, 2, Nk, 6))
    dof[:, :, :Nk - Nq] = 0.0
    dQf, dKf, dVf = _autograd(qf, k, v, dof, True, 0.45)
    dQ, dK, dV = attention_bwd_fp64(qf[:, :, Nk - Nq:], k, v, dof[:, :, Nk - Nq:], True, 0.45)
    assert np.abs(dQ - dQf[:, :, Nk - Nq:]).max() < 1e-12
    assert np.abs(dK - dKf).max() < 1e-12 and np.abs(dV - dVf).max() < 1e-12


@pytest.mark.parametrize("Nq,Nk", [(9, 1), (13, 4)])
def test_excess_queries_get_zero_gradient(Nq, Nk):
    g = np.random.default_rng(Nq + 5 * Nk)
    q, do = g.standard_normal((2, 1, 1, Nq, 6))
    k, v = g.standard_normal((2, 1, 1, Nk, 6))
    dQ, dK, dV = attention_bwd_fp64(q, k, v, do, True, 0.45)
    e = Nq - Nk
    assert np.all(dQ[:, :, :e] == 0.0)
    dQs, dKs, dVs = _autograd(q[:, :, e:], k, v, do[:, :, e:], True, 0.45)
    assert np.abs(dQ[:, :, e:] - dQs).max() < 1e-12
    assert np.abs(dK - dKs).max() < 1e-12 and np.abs(dV - dVs).max() < 1e-12


# ---- row chunking (bounded memory at long lengths) ------------------------------------------
@pytest.mark.parametrize("Nq,Nk,causal", [(23, 23, True), (23, 23, False), (17, 40, True),
                                          (40, 17, True), (33, 9, False)])
@pytest.mark.parametrize("chunk", [1, 5, 16])
def test_row_chunks_are_the_same_computation(Nq, Nk, causal, chunk):
    """Taking the query rows in chunks is the same computation (each row's P, dP and dS
    depend on that row alone; dK, dV sum over rows): the chunked result equals the
    one-chunk result (itself pinned by autograd above, and here for the square case), so
    a mistake in the chunk offsets (the mask shifted by the chunk start, a dropped or
    doubled chunk of dK / dV) fails here."""
    g = np.random.default_rng(Nq * 3 + Nk + chunk)
    q, do = g.standard_normal((2, 1, 2, Nq, 8))
    k, v = g.standard_normal((2, 1, 2, Nk, 8))
    got = attention_bwd_fp64(q, k, v, do, causal, 0.37, row_chunk=chunk)
    whole = attention_bwd_fp64(q, k, v, do, causal, 0.37, row_chunk=1 << 30)
    for a, b in zip(got, whole):
        assert np.abs(a - b).max() < 1e-12
    if Nq == Nk:
        for a, r in zip(got, _autograd(q, k, v, do, causal, 0.37)):
            assert np.abs(a - r).max() < 1e-11
