"""Parity of the backward pass (fa2_bwd through the C ABI) with the fp64 oracle.

Inputs Q, K, V and the upstream gradient dO are seeded bf16; O and L come from this library's
forward pass (as a caller would pass them).  The oracle (oracle/backward.py) computes dQ, dK, dV
from the same bf16 values by the plain chain rule in fp64.

Tolerance: max |g - g_ref| <= 2e-2 * max(1, max |g_ref|) for each of dQ, dK, dV.  The errors
are relative ones: P and dS enter their MFMA products rounded to bf16 (2^-9 relative), D =
rowsum(dO * O) is formed from the bf16 O, and each output is rounded to bf16 once, so a few
roundings of 2^-9 of the gradient's own size; 2e-2 is the forward's bound for O (whose values
stay below ~5.5 here), kept for gradients of magnitude <= 1 and scaled with the gradient
above that (peaked softmaxes, e.g. |scale| well above 1/sqrt(d), give gradients of 5 or
more).  The measured errors are printed.  Outputs are pre-filled with NaN.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from exact_attention_62_amd import FlashAttention, attention, attention_backward
from exact_attention_62_amd.inputs import make_random, make_upstream
from oracle.backward import attention_bwd_fp64

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def _say(msg):
    print(f"\n[bwd] {msg}", flush=True)
    sys.stdout.flush()


def _grad_inputs(B, H, N, d, seed):
    q, k, v = make_random(B, H, N, d, seed=seed)
    return q, k, v, make_upstream(B, H, N, d, seed=seed)


def _check(got, ref, what):
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        g64 = g.double().cpu().numpy()
        assert np.all(np.isfinite(g64)), f"{what}: non-finite {name}"
        e = float(np.abs(g64 - r).max())
        tol = TOL * max(1.0, float(np.abs(r).max()))
        errs.append(e)
        assert e <= tol, f"{what}: max |{name} - ref| = {e:.3e} > {tol:.3e} (max |ref| {np.abs(r).max():.2f})"
    _say(f"{what}: max err dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}")


SHAPES = [(1, 1, 1, 64), (1, 1, 7, 128), (1, 2, 64, 64), (2, 1, 127, 128), (1, 3, 129, 64),
          (1, 2, 200, 128), (2, 2, 300, 64), (1, 1, 513, 128), (1, 2, 1024, 128),
          # the other head dimensions: d = 32 and 96 stage their 32-query tiles in fewer 1 KB
          # loads than (or not a multiple of) the four wavefronts; d = 256 runs one workgroup
          # per CU
          (1, 1, 1, 32), (1, 2, 100, 32), (2, 1, 300, 32), (1, 1, 7, 96), (1, 2, 129, 96),
          (2, 1, 400, 96), (1, 1, 1, 256), (1, 2, 127, 256), (1, 1, 300, 256)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_matches_the_oracle(shape, causal):
    B, H, N, d = shape
    _say(f"B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v, do = _grad_inputs(B, H, N, d, seed=N + d + causal)
    ref = attention_bwd_fp64(q, k, v, do, causal=causal)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = attention(qd, kd, vd, causal=causal)
    got = attention_backward(qd, kd, vd, o, lse, dod, causal=causal)
    torch.cuda.synchronize()
    _check(got, ref, f"{shape} causal={causal}")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.3])
def test_bwd_zero_and_negative_scale(scale):
    q, k, v, do = _grad_inputs(1, 2, 160, 64, seed=77)
    ref = attention_bwd_fp64(q, k, v, do, causal=True, scale=scale)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = attention(qd, kd, vd, causal=True, scale=scale)
    _check(attention_backward(qd, kd, vd, o, lse, dod, causal=True, scale=scale), ref,
           f"scale={scale}")


def test_bwd_outputs_fully_written_and_deterministic():
    from exact_attention_62_amd import fa2_bwd, fa2_bwd_workspace_size
    q, k, v, do = (t.cuda() for t in _grad_inputs(2, 2, 333, 128, seed=5))
    o, lse = attention(q, k, v, causal=True)
    outs = []
    for _ in range(2):
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        ws = torch.full((fa2_bwd_workspace_size(2, 2, 333, 128) // 4,), float("nan"),
                        device="cuda")
        fa2_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert torch.isfinite(t.float()).all()
        outs.append((dq, dk, dv))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_autograd_wrapper():
    q, k, v, do = _grad_inputs(1, 2, 96, 64, seed=9)
    ref = attention_bwd_fp64(q, k, v, do, causal=True)
    qd, kd, vd = (t.cuda().requires_grad_() for t in (q, k, v))
    o = FlashAttention.apply(qd, kd, vd, True, None)
    o.backward(do.cuda())
    _check((qd.grad, kd.grad, vd.grad), ref, "autograd wrapper")


# ---- fp16 and query/key lengths that differ --------------------------------------------------
def _run_bwd(q, k, v, do, causal, scale=None):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = attention(qd, kd, vd, causal=causal, scale=scale)
    got = attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return got


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 64, 64), (2, 1, 127, 128), (1, 2, 300, 64),
                                   (1, 1, 513, 128), (1, 2, 200, 32), (1, 1, 129, 96),
                                   (1, 1, 130, 256)], ids=lambda s: "x".join(map(str, s)))
def test_bwd_fp16(shape, causal):
    B, H, N, d = shape
    _say(f"fp16 B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_random(B, H, N, d, seed=N + d + causal + 5, dtype="fp16")
    do = make_upstream(B, H, N, d, seed=N + d, dtype="fp16")
    ref = attention_bwd_fp64(q, k, v, do, causal=causal)
    _check(_run_bwd(q, k, v, do, causal), ref, f"fp16 {shape} causal={causal}")


CROSS = [
    # (B, H, Nq, Nk, d): short query blocks over long keys, one query, more queries than keys
    # (the first Nq - Nk rows see no key under the causal mask), ragged both ways, one key
    (1, 2, 5, 300, 64), (2, 1, 64, 200, 128), (1, 2, 1, 513, 128), (1, 2, 200, 64, 64),
    (1, 1, 300, 129, 128), (1, 2, 129, 1, 64), (2, 2, 100, 1000, 64),
    (1, 2, 70, 300, 32), (1, 1, 300, 129, 96), (1, 2, 50, 400, 256),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CROSS, ids=lambda c: "x".join(map(str, c)))
def test_bwd_cross_lengths(case, causal, dtype):
    B, H, Nq, Nk, d = case
    _say(f"cross {dtype} B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    q, k, v = make_random(B, H, Nq, d, seed=Nq + 3 * Nk + causal, dtype=dtype, Nk=Nk)
    do = make_upstream(B, H, Nq, d, seed=Nq + Nk, dtype=dtype)
    ref = attention_bwd_fp64(q, k, v, do, causal=causal)
    got = _run_bwd(q, k, v, do, causal)
    assert got[0].shape == q.shape and got[1].shape == k.shape and got[2].shape == v.shape
    _check(got, ref, f"cross {dtype} {case} causal={causal}")


def test_bwd_cross_no_queries_and_no_keys():
    from exact_attention_62_amd import fa2_bwd, fa2_bwd_workspace_size
    # No queries: dK = dV = 0 must still be written; no keys: dQ = 0.
    for Nq, Nk in ((0, 70), (70, 0)):
        q, k, v = (t.cuda() for t in make_random(1, 2, Nq, 64, seed=9, Nk=Nk))
        do = make_upstream(1, 2, Nq, 64, seed=9).cuda()
        o = torch.zeros_like(q)
        lse = torch.full((1, 2, Nq), float("-inf"), device="cuda")
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        ws = torch.empty(max(4, fa2_bwd_workspace_size(1, 2, Nq, 64)), dtype=torch.uint8,
                         device="cuda")
        fa2_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, causal=True)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert bool(torch.all(t == 0)), f"Nq={Nq} Nk={Nk}: not all zero"


def test_autograd_wrapper_cross_fp16():
    q, k, v = make_random(1, 2, 96, 64, seed=12, dtype="fp16", Nk=333)
    do = make_upstream(1, 2, 96, 64, seed=12, dtype="fp16")
    ref = attention_bwd_fp64(q, k, v, do, causal=True)
    qd, kd, vd = (t.cuda().requires_grad_() for t in (q, k, v))
    out = FlashAttention.apply(qd, kd, vd, True, None)
    out.backward(do.cuda())
    torch.cuda.synchronize()
    _check((qd.grad, kd.grad, vd.grad), ref, "autograd cross fp16")


# ------------------------------------------- the sizes the benchmark times, sampled heads
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("name", ["train", "long"])
def test_bwd_benchmark_shapes_sampled_heads(name, causal):
    """The backward pass at the sizes `bench.py --backward` times (16 x 16 x 2048 and
    1 x 16 x 16384, d = 128, bf16), launched on the whole problem, compared with the
    oracle on every element of dQ, dK and dV of four (batch, head) slices (the first, the
    last and two drawn at random)."""
    from exact_attention_62_amd.inputs import WORKLOADS, make

    w = WORKLOADS[name]
    B, H, N, d = w.B, w.H, w.N, w.d
    _say(f"backward {name} B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make(w, 0)
    do = make_upstream(B, H, N, d, 0)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = attention(qd, kd, vd, causal=causal, scale=w.scale)
    dq, dk, dv = attention_backward(qd, kd, vd, o, lse, dod, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    rng = np.random.default_rng(11 + causal)
    heads = sorted({(0, 0), (B - 1, H - 1)} | {(int(rng.integers(B)), int(rng.integers(H)))
                                                for _ in range(2)})
    while len(heads) < 4:  # draw again on a collision
        heads = sorted(set(heads) | {(int(rng.integers(B)), int(rng.integers(H)))})
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = attention_bwd_fp64(q[sl], k[sl], v[sl], do[sl], causal, w.scale, row_chunk=2048)
        _check((dq[sl], dk[sl], dv[sl]), ref, f"{name} head ({b},{h}) causal={causal}")
