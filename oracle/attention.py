"""fp64 CPU oracle for the FlashAttention-2 forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes
----------------
The FlashAttention-2 forward pass is exact attention computed tile by tile:
after the inner loop has visited every K/V block, the running result equals
the global softmax result (page "Flash Attention V2原理解读", commentary on
the FWD pseudo-code's inner loop).  So the oracle is that plain definition, written
out with the whole score row materialised, for every (batch, head):

    S[i, j] = scale * sum_k Q[i, k] * K[j, k]
    S[i, j] = -inf            where causal and j > i   (top-left aligned)
    m_i     = max_j S[i, j]
    P[i, j] = exp(S[i, j] - m_i)
    l_i     = sum_j P[i, j]
    O[i, :] = (sum_j P[i, j] * V[j, :]) / l_i
    L_i     = m_i + ln(l_i)

L is the single per-row statistic the method stores (page
"FlashAttention学习笔记(2)", section "V2 的运作流程 / forward", and page
"flash-attention123和ring-attention", 优化1).  The softmax scale multiplies
the logits and L is in the scaled-logit domain; the pages never name the
scale, that reading is ours.

Query and key lengths.  The grid on the pages is sized by the query length
alone (page "FlashAttention学习笔记(2)", section "V2中的thread blocks排布":
num_m_block from seqlen_q), so Q may have Nq rows while K and V have Nk.  The
pages fix no causal convention for Nq != Nk; the reading here aligns the mask
bottom-right, so that the last query sees every key:

    S[i, j] = -inf            where causal and j > i + (Nk - Nq)

which is the top-left rule above when Nq == Nk.  With Nq > Nk the first
Nq - Nk rows see no key at all; for such a row the sum over keys is empty,
so L_i = ln(0) = -inf, and O_i is taken as 0 (the softmax has no value there).

Inputs of any float dtype are upcast exactly to float64.  Rows are processed
in chunks; each row's softmax is independent, so chunking does not change the
definition.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_fp64", "attention_rows_fp64", "scaled_logits_fp64"]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: upcast exactly on the CPU
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def scaled_logits_fp64(q_rows, k, row_idx, causal, scale, offset: int = 0):
    """S for the given query rows against every key, with the causal mask applied.

    q_rows: [R, d] float64, k: [Nk, d] float64, row_idx: [R] absolute row positions.
    Key j is hidden from row i when j > i + offset (offset = Nk - Nq, 0 for Nq == Nk).
    """
    S = scale * (q_rows @ k.T)
    if causal:
        cols = np.arange(k.shape[0])[None, :]
        S = np.where(cols > np.asarray(row_idx)[:, None] + offset, -np.inf, S)
    return S


def _rows(q_rows, k, v, row_idx, causal, scale, offset=0):
    """The definition above for a set of rows of one (batch, head)."""
    S = scaled_logits_fp64(q_rows, k, row_idx, causal, scale, offset)
    O = np.zeros((S.shape[0], v.shape[1]))
    L = np.full(S.shape[0], -np.inf)
    if S.shape[1] == 0:
        return O, L
    m = S.max(axis=1)
    seen = np.isfinite(m)  # rows with at least one visible key
    P = np.exp(S[seen] - m[seen, None])
    l = P.sum(axis=1)
    O[seen] = (P @ v) / l[:, None]
    L[seen] = m[seen] + np.log(l)
    return O, L


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v one [B, H, Nk, d] shape")
    return q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.shape[3]


def attention_fp64(q, k, v, causal: bool = False, scale: float | None = None,
                   row_chunk: int = 2048):
    """Exact attention of q [B, H, Nq, d] over k, v [B, H, Nk, d].

    Returns (O [B,H,Nq,d], L [B,H,Nq]) in float64.  The causal mask is aligned
    bottom-right (key j hidden from row i when j > i + Nk - Nq).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, Nk, d = _shapes(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, Nq, d))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_chunk):
                r1 = min(Nq, r0 + row_chunk)
                O[b, h, r0:r1], L[b, h, r0:r1] = _rows(
                    q[b, h, r0:r1], k[b, h], v[b, h], np.arange(r0, r1), causal, scale, Nk - Nq)
    return O, L


def attention_rows_fp64(q, k, v, b: int, h: int, rows, causal: bool = False,
                        scale: float | None = None):
    """The same definition for selected rows of one (batch, head) of a large problem.

    ``q`` ([B, H, Nq, d]), ``k`` and ``v`` ([B, H, Nk, d]) may be torch tensors or
    arrays; only head (b, h) is upcast.  Returns (O [R, d], L [R]) in float64.
    """
    qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
    d = qh.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.asarray(rows, dtype=np.int64)
    return _rows(qh[rows], kh, vh, rows, causal, scale, kh.shape[0] - qh.shape[0])
