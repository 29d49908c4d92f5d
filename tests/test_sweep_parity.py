"""Property sweep of small shapes, and independence of the work order.

Sweep: the forward pass through the C ABI (fa2_fwd_cross, which fa2_fwd is the Nq = Nk case
of) against the fp64 oracle on shapes hypothesis draws: B in 1..2, H in 1..3, Nq and Nk in
1..300, every head dimension the kernels build (32, 64, 96, 128, 256), bf16 or fp16, with or
without the causal mask (aligned bottom-right).  The draw is derandomized, so every run checks
the same cases.  Tolerances as in the other parity tests (max-abs: bf16 O 2e-2, L 1e-3; fp16
O 1e-2, L 1e-3); outputs start as NaN so an element not written fails.

Work order: each output row depends only on its own (batch, head) slice and query block
(page "FlashAttention学习笔记(2)", section "V2中的thread blocks排布": one independent block of
work per query block, batch and head).  Permuting the heads of the input hands every work
item to another workgroup, at another position of its sequence (and so with other LDS
buffers), so the permuted outputs must be the original outputs permuted, bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from exact_attention_62_amd import attention, fa2_fwd_cross
from exact_attention_62_amd.inputs import make_random
from oracle import attention_fp64

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "fp16": (1e-2, 1e-3)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _say(msg):
    print(f"\n[sweep] {msg}", flush=True)
    sys.stdout.flush()


@settings(max_examples=150, derandomize=True, deadline=None, database=None,
          suppress_health_check=list(HealthCheck))
@given(B=st.integers(1, 2), H=st.integers(1, 3), Nq=st.integers(1, 300),
       Nk=st.one_of(st.none(), st.integers(1, 300)),
       d=st.sampled_from([32, 64, 96, 128, 256]), dtype=st.sampled_from(["bf16", "fp16"]),
       causal=st.booleans(), seed=st.integers(0, 2**16))
def test_small_shapes_against_the_oracle(B, H, Nq, Nk, d, dtype, causal, seed):
    Nk = Nq if Nk is None else Nk
    _say(f"{dtype} B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} seed={seed}")
    q, k, v = make_random(B, H, Nq, d, seed=seed, dtype=dtype, Nk=Nk)
    O, L = attention_fp64(q, k, v, causal=causal)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    fa2_fwd_cross(qd, kd, vd, o, lse, causal=causal)
    torch.cuda.synchronize()
    o64, l64 = o.double().cpu().numpy(), lse.double().cpu().numpy()
    none = np.isneginf(L)
    assert np.array_equal(np.isneginf(l64), none)
    assert np.all(np.isfinite(o64)) and np.all(o64[none] == 0.0)
    otol, ltol = TOL[dtype]
    assert np.abs(o64 - O).max() <= otol
    if (~none).any():
        assert np.abs(l64[~none] - L[~none]).max() <= ltol


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 40, 1000, 128, True),    # more items than the grid: several per workgroup
    (2, 16, 777, 64, True),
    (1, 24, 600, 256, False),
])
def test_permuting_heads_permutes_the_outputs_bitwise(B, H, N, d, causal):
    _say(f"permuted heads B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = (t.cuda() for t in make_random(B, H, N, d, seed=H * N + d, dtype="bf16"))
    o, lse = attention(q, k, v, causal=causal)
    g = torch.Generator().manual_seed(N + d)
    perm = torch.randperm(H, generator=g).cuda()
    op, lp = attention(q[:, perm].contiguous(), k[:, perm].contiguous(), v[:, perm].contiguous(),
                       causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(op, o[:, perm]) and torch.equal(lp, lse[:, perm])
