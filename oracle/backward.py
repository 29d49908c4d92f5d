"""fp64 CPU oracle for the FlashAttention-2 backward pass (gradients of O with respect to Q, K, V).

TEST INFRASTRUCTURE ONLY (see oracle/attention.py): imported by the tests, never by the
library, and sharing no code with the HIP path.

What the pages fix (page "FlashAttention学习笔记(2)", the forward section and "Foward和backward
中的thread block划分"; page "Flash Attention V2原理解读", the backward discussion; page
"flash-attention123和ring-attention", 优化1):
  * the backward recomputes S and P block by block instead of storing them;
  * it needs only the per-row statistic L = m + ln(l) from the forward: with L in place of the
    row max, exp(S - L) is already the normalised softmax weight P;
  * its loops are KV outer, Q inner: dK and dV accumulate along a KV block's rows, dQ across KV
    blocks.
The gradient formulas themselves did not survive on the pages (they defer to the V1
derivation).  The reading here is the plain chain rule of softmax attention, which is what the
method reaches exactly (up to rounding order), so the oracle is that definition written out:

    P  = softmax(scale * Q K^T, causal mask)           (each row; masked entries 0)
    dV = P^T dO
    dP = dO V^T
    D  = rowsum(dO * O)  (= rowsum(P * dP), since O = P V)
    dS = P * (dP - D)                                   (elementwise, D broadcast along rows)
    dQ = scale * dS K
    dK = scale * dS^T Q

computed per (batch, head) with the whole score matrix materialised, in float64.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_bwd_fp64", "delta_fp64"]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _probs(q_rows, k, rows, causal, scale, offset):
    """Row softmax of the masked logits of the given query rows (absolute positions
    `rows`; key j is hidden from row i when j > i + offset); a row that sees no key has
    P = 0."""
    Nk = k.shape[0]
    S = scale * (q_rows @ k.T)
    if causal:
        S = np.where(np.arange(Nk)[None, :] > np.asarray(rows)[:, None] + offset, -np.inf, S)
    P = np.zeros_like(S)
    if Nk == 0:
        return P
    m = S.max(axis=1, keepdims=True)
    seen = np.isfinite(m[:, 0])
    P[seen] = np.exp(S[seen] - m[seen])
    P[seen] /= P[seen].sum(axis=1, keepdims=True)
    return P


def delta_fp64(o, do):
    """D[b, h, i] = sum_k dO[b, h, i, k] * O[b, h, i, k]."""
    return (_f64(o) * _f64(do)).sum(axis=-1)


def attention_bwd_fp64(q, k, v, do, causal: bool = False, scale: float | None = None,
                       row_chunk: int = 2048):
    """(dQ [B,H,Nq,d], dK, dV [B,H,Nk,d]) in float64, for O = attention(q, k, v) and upstream dO.

    q and do are [B, H, Nq, d], k and v [B, H, Nk, d]; the causal mask is aligned
    bottom-right as in the forward oracle, and rows that see no key (P = 0) add nothing.
    Query rows are taken in chunks of at most `row_chunk` (each row's P, dP and dS depend on
    that row alone; dK and dV are sums over rows), which bounds the memory at long lengths.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_chunk):
                r1 = min(Nq, r0 + row_chunk)
                P = _probs(q[b, h, r0:r1], k[b, h], np.arange(r0, r1), causal, scale, Nk - Nq)
                O = P @ v[b, h]
                dV[b, h] += P.T @ do[b, h, r0:r1]
                dP = do[b, h, r0:r1] @ v[b, h].T
                D = (do[b, h, r0:r1] * O).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                dQ[b, h, r0:r1] = scale * (dS @ k[b, h])
                dK[b, h] += scale * (dS.T @ q[b, h, r0:r1])
    return dQ, dK, dV
