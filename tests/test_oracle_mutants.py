"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and check that at least one pin catches it."""
import math

import pytest
import torch

from tests import oracle_pins


def _make(head_fn, raw_scale=False):
    def attn(q, k, v, scale):
        # raw_scale plants the mistake of using the scale without its float32 rounding
        sigma = scale if raw_scale else float(torch.tensor(scale, dtype=torch.float32).item())
        B, H, Sq, _ = q.shape
        o = torch.empty((B, H, Sq, v.shape[3]), dtype=torch.float64)
        lse = torch.empty((B, H, Sq), dtype=torch.float64)
        for b in range(B):
            for h in range(H):
                o[b, h], lse[b, h] = head_fn(q[b, h].double(), k[b, h].double(), v[b, h].double(), sigma)
        return o, lse
    return attn


def _ok(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp(s - m)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, m.squeeze(1) + torch.log(l.squeeze(1))


def _no_scale(qd, kd, vd, sigma):
    return _ok(qd, kd, vd, 1.0)


def _scale_squared(qd, kd, vd, sigma):
    return _ok(qd, kd, vd, sigma * sigma)


def _lse_log2(qd, kd, vd, sigma):
    o, lse = _ok(qd, kd, vd, sigma)
    return o, lse / math.log(2.0)


def _lse_without_max(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp(s - m)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, torch.log(l.squeeze(1))


def _no_max_trick(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    e = torch.exp(s)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, torch.log(l.squeeze(1))


def _no_normalise(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp(s - m)
    l = e.sum(dim=1, keepdim=True)
    return e @ vd, m.squeeze(1) + torch.log(l.squeeze(1))


def _exp2_instead_of_exp(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp2(s - m)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, m.squeeze(1) + torch.log(l.squeeze(1))


def _sign_flip(qd, kd, vd, sigma):
    s = (qd @ kd.T) * sigma
    m = s.min(dim=1, keepdim=True).values
    e = torch.exp(m - s)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, -m.squeeze(1) + torch.log(l.squeeze(1))


def _transposed_scores(qd, kd, vd, sigma):
    # softmax over the query axis instead of the key axis (square cases only)
    s = (qd @ kd.T) * sigma
    if s.shape[0] != s.shape[1]:
        s = s[:, : s.shape[0]] if s.shape[1] > s.shape[0] else torch.nn.functional.pad(s, (0, s.shape[0] - s.shape[1]))
        vd = vd[: s.shape[1]] if vd.shape[0] >= s.shape[1] else torch.nn.functional.pad(vd, (0, 0, 0, s.shape[1] - vd.shape[0]))
    st = s.T
    m = st.max(dim=1, keepdim=True).values
    e = torch.exp(st - m)
    l = e.sum(dim=1, keepdim=True)
    return (e @ vd) / l, m.squeeze(1) + torch.log(l.squeeze(1))


def _drop_last_key(qd, kd, vd, sigma):
    if kd.shape[0] > 1:
        kd, vd = kd[:-1], vd[:-1]
    return _ok(qd, kd, vd, sigma)


def _sum_of_unshifted(qd, kd, vd, sigma):
    # row sum taken before subtracting the max, numerator after
    s = (qd @ kd.T) * sigma
    m = s.max(dim=1, keepdim=True).values
    e = torch.exp(s - m)
    l = torch.exp(s).sum(dim=1, keepdim=True)
    return (e @ vd) / l, m.squeeze(1) + torch.log(e.sum(dim=1))


def _mean_instead_of_sum(qd, kd, vd, sigma):
    o, lse = _ok(qd, kd, vd, sigma)
    return o, lse - math.log(kd.shape[0])


MUTANTS = [_no_scale, _scale_squared, _lse_log2, _lse_without_max, _no_max_trick, _no_normalise,
           _exp2_instead_of_exp, _sign_flip, _transposed_scores, _drop_last_key, _sum_of_unshifted,
           _mean_instead_of_sum]


def _caught(attn, pins=oracle_pins.ALL_PINS):
    for pin in pins:
        try:
            pin(attn)
        except (AssertionError, RuntimeError, IndexError, ValueError):
            return pin.__name__
    return None


def test_reference_copy_passes_all_pins():
    assert _caught(_make(_ok)) is None


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_mutant_is_caught(mutant):
    assert _caught(_make(mutant)) is not None, f"no pin catches {mutant.__name__}"


def test_unrounded_scale_is_caught():
    """A copy that uses the scale as given instead of its float32 value."""
    assert _caught(_make(_ok, raw_scale=True)) == "pin_inexact_scale"


# ---- mutants of the probability matrix ----

def _sigma(scale):
    return float(torch.tensor(scale, dtype=torch.float32).item())


def _probs_ok(q, k, scale):
    s = (q.double() @ k.double().transpose(-1, -2)) * _sigma(scale)
    e = torch.exp(s - s.max(dim=-1, keepdim=True).values)
    return e / e.sum(dim=-1, keepdim=True)


def _probs_no_scale(q, k, scale):
    return _probs_ok(q, k, 1.0)


def _probs_raw_scale(q, k, scale):
    s = (q.double() @ k.double().transpose(-1, -2)) * scale
    e = torch.exp(s - s.max(dim=-1, keepdim=True).values)
    return e / e.sum(dim=-1, keepdim=True)


def _probs_exp2(q, k, scale):
    s = (q.double() @ k.double().transpose(-1, -2)) * _sigma(scale)
    e = torch.exp2(s - s.max(dim=-1, keepdim=True).values)
    return e / e.sum(dim=-1, keepdim=True)


def _probs_over_queries(q, k, scale):
    s = (q.double() @ k.double().transpose(-1, -2)) * _sigma(scale)
    e = torch.exp(s - s.max(dim=-2, keepdim=True).values)
    return e / e.sum(dim=-2, keepdim=True)


def _probs_no_max_trick(q, k, scale):
    e = torch.exp((q.double() @ k.double().transpose(-1, -2)) * _sigma(scale))
    return e / e.sum(dim=-1, keepdim=True)


def _probs_unnormalised(q, k, scale):
    s = (q.double() @ k.double().transpose(-1, -2)) * _sigma(scale)
    return torch.exp(s - s.max(dim=-1, keepdim=True).values)


PROB_MUTANTS = [_probs_no_scale, _probs_raw_scale, _probs_exp2, _probs_over_queries,
                _probs_no_max_trick, _probs_unnormalised]


def test_reference_probs_copy_passes():
    assert _caught(_probs_ok, oracle_pins.PROB_PINS) is None


@pytest.mark.parametrize("mutant", PROB_MUTANTS, ids=lambda m: m.__name__)
def test_probs_mutant_is_caught(mutant):
    assert _caught(mutant, oracle_pins.PROB_PINS) is not None, f"no pin catches {mutant.__name__}"
