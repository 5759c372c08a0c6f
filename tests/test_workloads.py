"""Seeded input generators (no GPU)."""
import torch

import workloads
from workloads import WORKLOADS, make_inputs, make_random


def test_workload_table():
    assert [w.name for w in WORKLOADS] == ["s256", "s1k", "s4k", "s8k_peaked", "s16k_outliers"]
    assert [(w.B, w.H, w.S, w.D) for w in WORKLOADS] == [
        (1, 1, 256, 128), (2, 16, 1024, 128), (4, 16, 4096, 128), (2, 16, 8192, 128), (1, 16, 16384, 128)]
    assert [w.seed for w in WORKLOADS] == [1001, 1002, 1003, 1004, 1005]
    assert all(w.scale == float(torch.tensor(128 ** -0.5, dtype=torch.float32)) for w in WORKLOADS)
    assert WORKLOADS[4].flops == 4 * 16 * 16384 * 16384 * 128


def test_deterministic_and_shaped():
    w = workloads.get("s1k")
    a = make_inputs(w, B=1, H=2, S=256)
    b = make_inputs(w, B=1, H=2, S=256)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 256, 128) and x.is_contiguous()
        assert torch.equal(x, y)
    c = make_inputs(workloads.get("s4k"), B=1, H=2, S=256)
    assert not torch.equal(a[0], c[0])


def test_distributions():
    q, k, v = make_inputs(workloads.get("s8k_peaked"), B=1, H=2, S=2048)
    assert abs(q.float().std().item() - 2.0) < 0.02 and abs(k.float().std().item() - 2.0) < 0.02
    assert v.float().min().item() >= -1.0 and v.float().max().item() <= 1.0
    assert abs(v.float().mean().item()) < 0.01
    q, k, v = make_inputs(workloads.get("s4k"), B=1, H=2, S=2048)
    for t in (q, k, v):
        assert abs(t.float().std().item() - 1.0) < 0.01


def test_outlier_rows():
    """Exactly round(1% of S) K rows per (b, h) are 8x the plain draw."""
    w = workloads.get("s16k_outliers")
    S = 2048
    q, k, v = make_inputs(w, B=1, H=3, S=S)
    plain = workloads.Workload("plain", w.index, 1, 3, S, 128, "normal", 1.0, "normal", 0.0, 1.0, w.scale)
    q0, k0, v0 = make_inputs(plain)
    assert torch.equal(q, q0) and torch.equal(v, v0)
    n = workloads.outlier_rows(S, 0.01)
    assert n == 20 and workloads.outlier_rows(16384, 0.01) == 164
    for h in range(3):
        diff = (k[0, h] != k0[0, h]).any(dim=1)
        rows = diff.nonzero().flatten()
        assert len(rows) <= n
        # rows whose draw is exactly zero in every dim could hide; none are here
        assert len(rows) == n
        assert torch.equal(k[0, h, rows].float(), k0[0, h, rows].float() * 8)


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], dtype=torch.float32)
    y = x.to(torch.bfloat16).float()
    assert y.tolist() == [1.0, 1.0 + 2 ** -6, -1.0]


def test_make_random_matches_recipe():
    q, k, v = make_random(1, 1, 128, 128, seed=1003)
    q2, k2, v2 = make_inputs(workloads.get("s4k"), B=1, H=1, S=128)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
