"""fp64 CPU model of the FlashAttention-2 forward algorithm, tile by tile.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).  It exists to pin the
claim the whole method rests on: that the tiled loop with an online running
max and sum reaches exactly the plain attention result.  It follows the
algorithm in the pages' order and notation:

  * outer loop over query blocks Q_i of Br rows; the block's running O_i,
    m_i, l_i stay local for the whole inner loop (page "FlashAttention学习笔记(2)",
    opening section; page "Flash Attention V2原理解读", FWD commentary);
  * inner loop over key/value blocks K_j, V_j of Bc rows:
      - the score block S_i^(j) = scale * Q_i K_j^T
      - the softmax update: m_i^(j) = max(m_i^(j-1), rowmax S_i^(j)),
        P~ = exp(S_i^(j) - m_i^(j)),
        l_i^(j) = exp(m_i^(j-1) - m_i^(j)) l_i^(j-1) + rowsum P~
      - the output update: O_i^(j) = diag(exp(m_i^(j-1) - m_i^(j))) O_i^(j-1)
        + P~ V_j, with no division by l inside the loop
  * after the loop, O_i = diag(l_i)^-1 O_i once and L_i = m_i + log(l_i)
    (page "FlashAttention学习笔记(2)", forward; page
    "flash-attention123和ring-attention", 优化1 and 优化2);
  * with the causal mask, K/V blocks that lie entirely above the diagonal
    are skipped, not computed and then masked (page
    "flash-attention123和ring-attention", 优化3).

The text of the pseudo-code's inner-loop steps did not survive on the pages; the steps
above are rebuilt from the surviving prose plus the online-softmax
mathematics.  ``deferred_norm=False`` gives the per-step normalised variant
(dividing by the running l every step) that 优化2 says the deferral removes;
``skip_masked=False`` computes every block and relies on the mask alone.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["fa2_forward_tiled_fp64", "causal_block_end"]


def causal_block_end(i: int, Br: int, Bc: int, N: int) -> int:
    """Number of K/V blocks query block i must visit under the causal mask.

    Block j is entirely masked for query block i when its first key lies
    after the block's last row, min(N, (i+1)*Br) - 1.
    """
    last_row = min(N, (i + 1) * Br) - 1
    return last_row // Bc + 1


def fa2_forward_tiled_fp64(q, k, v, causal: bool = False, scale: float | None = None,
                           Br: int = 64, Bc: int = 64, deferred_norm: bool = True,
                           skip_masked: bool = True):
    """Tiled forward pass on [B, H, N, d] float arrays.  Returns (O, L) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    Tr = -(-N // Br)
    Tc = -(-N // Bc)
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(Tr):
                r0, r1 = i * Br, min(N, (i + 1) * Br)
                Qi = q[b, h, r0:r1]
                rows = np.arange(r0, r1)
                Oi = np.zeros((r1 - r0, d))
                li = np.zeros(r1 - r0)
                mi = np.full(r1 - r0, -np.inf)
                j_end = causal_block_end(i, Br, Bc, N) if (causal and skip_masked) else Tc
                for j in range(j_end):
                    c0, c1 = j * Bc, min(N, (j + 1) * Bc)
                    Kj, Vj = k[b, h, c0:c1], v[b, h, c0:c1]
                    S = scale * (Qi @ Kj.T)  # score block
                    if causal:
                        S = np.where(np.arange(c0, c1)[None, :] > rows[:, None], -np.inf, S)
                    m_new = np.maximum(mi, S.max(axis=1))
                    # A row that has seen only masked keys keeps m = -inf; shift by 0
                    # there so that exp(-inf - (-inf)) never forms a NaN.
                    shift = np.where(np.isneginf(m_new), 0.0, m_new)
                    P = np.exp(S - shift[:, None])
                    alpha = np.exp(mi - shift)
                    l_new = alpha * li + P.sum(axis=1)  # running sum
                    if deferred_norm:
                        Oi = alpha[:, None] * Oi + P @ Vj  # output update, unnormalised
                    else:
                        Oi = ((alpha * li)[:, None] * Oi + P @ Vj) / l_new[:, None]
                    mi, li = m_new, l_new
                if deferred_norm:
                    Oi = Oi / li[:, None]  # normalise once
                O[b, h, r0:r1] = Oi
                L[b, h, r0:r1] = mi + np.log(li)  # logsumexp
    return O, L
