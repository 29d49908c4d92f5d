"""The seeded input recipe: deterministic, the stated shapes and distributions."""
import torch

from exact_attention_62_amd.inputs import WORKLOADS, make, make_random


def test_seeded_inputs_are_deterministic_and_distinct():
    a = make("small", 0, N=64)
    b = make("small", 0, N=64)
    c = make("small", 1, N=64)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    assert not torch.equal(a[0], a[1])  # Q, K, V are separate draws


def test_workload_shapes_and_dtypes():
    assert [w.name for w in sorted(WORKLOADS.values(), key=lambda w: w.index)] == [
        "tiny", "small", "train", "long", "ragged"]
    q, k, v = make("tiny", 0)
    assert q.shape == (1, 1, 128, 64) and q.dtype == torch.float32
    q, k, v = make("ragged", 0, B=1, H=1, N=300)
    assert q.dtype == torch.bfloat16 and q.shape == (1, 1, 300, 256)
    assert 3.0 < q.float().std().item() < 5.0  # N(0, sigma=4)
    assert v.float().abs().max().item() <= 1.0  # U(-1, 1)
    assert WORKLOADS["train"].flops(True) == 2.0 * 16 * 16 * 2048 * 2048 * 128


def test_make_random_shapes():
    q, k, v = make_random(2, 3, 17, 64, seed=5)
    assert q.shape == (2, 3, 17, 64) and v.dtype == torch.bfloat16
    assert q.is_contiguous() and k.is_contiguous() and v.is_contiguous()


def test_make_upstream_is_seeded_and_independent_of_the_inputs():
    from exact_attention_62_amd.inputs import make_random, make_upstream
    a = make_upstream(1, 2, 33, 64, seed=3)
    assert a.shape == (1, 2, 33, 64) and a.dtype == torch.bfloat16
    assert torch.equal(a, make_upstream(1, 2, 33, 64, seed=3))
    assert not torch.equal(a, make_upstream(1, 2, 33, 64, seed=4))
    q, _, _ = make_random(1, 2, 33, 64, seed=3)
    assert not torch.equal(a, q)
