"""The CPU oracle against its pins (no GPU)."""
import math

import pytest
import torch

import oracle
from oracle import attention_ref
from tests import oracle_pins
from workloads import DEFAULT_SCALE, make_random


def _attn(q, k, v, scale):
    return oracle.attention(q, k, v, scale)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_attn)


def test_small_blocks_match_one_block():
    """Blocking over query rows must not change anything."""
    q, k, v = make_random(1, 2, 256, 128, seed=2001)
    o1, l1 = oracle.attention(q, k, v, DEFAULT_SCALE, block_rows=1024)
    o2, l2 = oracle.attention(q, k, v, DEFAULT_SCALE, block_rows=48)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("pin", oracle_pins.PROB_PINS, ids=lambda p: p.__name__)
def test_probs_pin(pin):
    pin(oracle.attention_probs)


def test_probs_times_v_is_attention():
    """The probability matrix and the two-pass attention agree: P.V = O, and
    the log of each row's largest-P denominator matches lse (P_max = e^(s_max - lse))."""
    q, k, v = make_random(1, 2, 128, 128, seed=2005, qk_std=2.0)
    p = oracle.attention_probs(q, k, DEFAULT_SCALE)
    o, lse = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert (p @ v.double() - o).abs().max().item() < 1e-13
    s = (q.double() @ k.double().transpose(-1, -2)) * oracle.sigma_of(DEFAULT_SCALE)
    m = s.max(dim=-1).values
    assert (torch.log(p.max(dim=-1).values) - (m - lse)).abs().max().item() < 1e-12


def test_rows_of_p_sum_to_one():
    q, k, _ = make_random(1, 2, 128, 128, seed=2002, qk_std=2.0)
    p = oracle.attention_probs(q, k, DEFAULT_SCALE)
    assert (p >= 0).all()
    assert torch.allclose(p.sum(-1), torch.ones(p.shape[:-1], dtype=torch.float64), atol=1e-14, rtol=0)


def test_attention_rows_equals_full():
    q, k, v = make_random(2, 2, 256, 128, seed=2003)
    o, lse = oracle.attention(q, k, v, DEFAULT_SCALE)
    picks = [(0, 0, 0), (1, 1, 255), (0, 1, 17), (1, 0, 128), (0, 0, 5)]
    o2, l2 = oracle.attention_rows(q, k, v, DEFAULT_SCALE, picks)
    for n, (b, h, i) in enumerate(picks):
        assert torch.allclose(o2[n], o[b, h, i], atol=1e-14, rtol=0)
        assert abs(float(l2[n] - lse[b, h, i])) < 1e-12


def test_scale_is_rounded_to_float32():
    """The oracle uses the float32 value of the scale, as the kernel receives it."""
    s = 1.0 / math.sqrt(128)
    assert attention_ref.sigma_of(s) == float(torch.tensor(s, dtype=torch.float32))
    assert attention_ref.sigma_of(s) != s
    assert DEFAULT_SCALE == attention_ref.sigma_of(s)


def test_bf16_inputs_are_widened_exactly():
    q, k, v = make_random(1, 1, 128, 128, seed=2004)
    o1, l1 = oracle.attention(q, k, v, DEFAULT_SCALE)
    o2, l2 = oracle.attention(q.double(), k.double(), v.double(), DEFAULT_SCALE)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bad_shapes_rejected():
    q = torch.zeros((1, 1, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention(q, torch.zeros((1, 1, 4, 7)), torch.zeros((1, 1, 4, 8)), 1.0)
    with pytest.raises(ValueError):
        oracle.attention(q, torch.zeros((1, 2, 4, 8)), torch.zeros((1, 2, 4, 8)), 1.0)
