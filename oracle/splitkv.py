"""fp64 CPU oracle for attention split along the key/value sequence.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py): imported by the tests,
never by the library, and sharing no code with the HIP path.

What the pages say (page "Flash Attention V2原理解读", the thread-block grid
section): the key/value sequence can also be split across thread blocks, but
then the blocks are no longer independent: each row of O gets one part from
every split, and the parts must be combined once more to reach the global
softmax result.  The pages recommend it only when the query-block grid cannot
fill the GPU, and choose the number of splits with a heuristic: compute the
utilisation for each candidate number of splits, take the highest, and pick
the smallest candidate whose utilisation is at least 0.95 of it.

What this module computes
-------------------------
* ``attention_keyrange_fp64``: the plain attention definition restricted to the
  keys in [lo, hi) of each row: for each row the partial output
  O_s = sum_j P_j V_j / l_s (normalised within the range) and
  L_s = m_s + ln(l_s).  A row with no visible key in the range has no softmax:
  O_s = 0 and L_s = -inf.
* ``combine_fp64``: the merge of partial results.  From the definition,
  exp(L_s) = sum_{j in s} exp(S_j) is each range's share of the row's softmax
  denominator, so L = ln sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s.
  Ranges with L_s = -inf contribute nothing.
* ``num_splits_heuristic``: the pages' selection rule.  The pages do not
  define "utilisation"; the reading here is the fraction of the last round of
  work that keeps the GPU busy: with n work units over `slots` concurrent
  slots, util = (n / slots) / ceil(n / slots).  The candidates are
  1..max_splits.
* ``split_ranges``: one way of cutting B KV blocks into s contiguous ranges
  (ceil(B/s) blocks each, the last ones possibly short or empty); the combine
  result does not depend on the cut.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_keyrange_fp64", "combine_fp64", "num_splits_heuristic", "split_ranges",
           "utilisation"]


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_keyrange_fp64(q, k, v, lo: int, hi: int, causal: bool = False,
                            scale: float | None = None):
    """Partial attention over keys [lo, hi) of every row: (O_s [B,H,Nq,d], L_s [B,H,Nq]).

    q is [B, H, Nq, d], k and v [B, H, Nk, d].  Plain definition per row (no
    tiling): S = scale * q k^T over the keys in the range, the causal mask hides
    keys j > i + Nk - Nq (bottom-right aligned), then m, P = exp(S - m), l,
    O = P V / l, L = m + ln l.  Rows with no visible key: O = 0, L = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, Nq, d))
    L = np.full((B, H, Nq), -np.inf)
    lo, hi = max(0, lo), min(Nk, hi)
    if hi <= lo:
        return O, L
    keys = np.arange(lo, hi)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h, lo:hi].T)  # [Nq, hi-lo]
            if causal:
                S = np.where(keys[None, :] > np.arange(Nq)[:, None] + (Nk - Nq), -np.inf, S)
            m = S.max(axis=1)
            seen = np.isfinite(m)
            P = np.exp(S[seen] - m[seen, None])
            l = P.sum(axis=1)
            O[b, h, seen] = (P @ v[b, h, lo:hi]) / l[:, None]
            L[b, h, seen] = m[seen] + np.log(l)
    return O, L


def combine_fp64(O_parts, L_parts):
    """Merge partial results: O_parts [S,...,d], L_parts [S,...] -> (O [...,d], L [...]).

    L = ln sum_s exp(L_s) (evaluated as max + ln sum exp(L_s - max)) and
    O = sum_s exp(L_s - L) O_s.  A row whose every L_s is -inf saw no key in any
    range: its sum is empty, L = -inf and O = 0.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    L_parts = np.asarray(L_parts, dtype=np.float64)
    Lmax = L_parts.max(axis=0)
    seen = np.isfinite(Lmax)
    ref = np.where(seen, Lmax, 0.0)
    w = np.exp(L_parts - ref[None])  # exp(-inf) = 0 for empty ranges
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(seen, ref + np.log(tot), -np.inf)
        O = np.where(seen[..., None], (w[..., None] * O_parts).sum(axis=0) / tot[..., None], 0.0)
    return O, L


def utilisation(units: int, slots: int) -> float:
    """Busy fraction of the last round: (units/slots) / ceil(units/slots)."""
    waves = units / slots
    return waves / math.ceil(waves)


def num_splits_heuristic(items: int, slots: int, max_splits: int) -> int:
    """The pages' rule: the smallest s in 1..max_splits with
    utilisation(items*s, slots) >= 0.95 * max over s of utilisation(items*s, slots)."""
    cands = range(1, max(1, max_splits) + 1)
    util = {s: utilisation(items * s, slots) for s in cands}
    best = max(util.values())
    return min(s for s in cands if util[s] >= 0.95 * best)


def split_ranges(n_blocks: int, s: int):
    """[(first, end), ...]: s contiguous ranges of ceil(n_blocks/s) blocks (some may be empty)."""
    per = -(-n_blocks // s)
    return [(min(i * per, n_blocks), min((i + 1) * per, n_blocks)) for i in range(s)]
