"""The tile-by-tile model of the article's online softmax (lazy rescale,
base-2 exponent, flush to zero) against the two-pass oracle and the values
the article prints (no GPU)."""
import json
import math
from pathlib import Path

import pytest
import torch

import oracle
from oracle import online_model
from workloads import DEFAULT_SCALE, dominant_key_small_lse_case, make_random

GOLDEN = json.loads((Path(__file__).parent / "golden" / "page_values.json").read_text())


def _val(name):
    return next(v for v in GOLDEN["values"] if v["name"] == name)


def test_page_values():
    t = _val("rebase_threshold_log2")
    assert online_model.REBASE_THRESH_LOG2 == t["value"]
    v = _val("peak_unnormalised_p_at_threshold")
    assert online_model.unnormalised_peak(v["log2_gap"]) == v["value"]
    v = _val("natural_gap_at_threshold")
    assert abs(online_model.natural_gap(v["log2_gap"]) - v["value"]) <= v["abs_tol"]
    v = _val("raw_qk_gap_at_threshold_hd128")
    assert abs(online_model.raw_score_gap(v["log2_gap"], v["head_dim"]) - v["value"]) <= v["abs_tol"]
    v = _val("worked_example_skip")
    assert abs(online_model.unnormalised_peak(v["log2_gap"]) - v["value"]) <= v["abs_tol"]
    v = _val("stale_base_gap_20")
    assert online_model.unnormalised_peak(v["log2_gap"]) == v["value"]


def _two_tile_case(gap_log2, block_n=4):
    """One query (D=1, q=1) over two tiles of block_n keys: tile 1 scores are
    all 0, tile 2 holds one key whose base-2 scaled score is gap_log2."""
    sigma = oracle.sigma_of(DEFAULT_SCALE)
    c = sigma * online_model.LOG2E
    k = torch.zeros((1, 1, 2 * block_n, 1), dtype=torch.float64)
    k[0, 0, block_n] = gap_log2 / c
    q = torch.ones((1, 1, 1, 1), dtype=torch.float64)
    v = torch.arange(2 * block_n, dtype=torch.float64).reshape(1, 1, 2 * block_n, 1)
    return q, k, v


def test_worked_example_no_rebase_below_threshold():
    """Gap 7.78 < 8: the kept base stays, the new key's P is ~219, and the
    result still equals the two-pass definition."""
    q, k, v = _two_tile_case(_val("worked_example_skip")["log2_gap"])
    stats = {}
    o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_m=1, block_n=4, stats=stats)
    assert stats["rebases"] == 0
    assert abs(stats["max_p"] - _val("worked_example_skip")["value"]) <= _val("worked_example_skip")["abs_tol"]
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_gap_20_rebases():
    """Gap 20 >= 8: the model rebases, so P never reaches 2^20."""
    q, k, v = _two_tile_case(_val("stale_base_gap_20")["log2_gap"])
    stats = {}
    o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_m=1, block_n=4, stats=stats)
    assert stats["rebases"] == 1
    assert stats["max_p"] <= 2.0 ** 8
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert torch.allclose(o, o_ref, atol=1e-12, rtol=0)
    assert torch.allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_never_rebasing_would_reach_2_pow_20():
    q, k, v = _two_tile_case(20.0)
    stats = {}
    online_model.online_attention(q, k, v, DEFAULT_SCALE, block_m=1, block_n=4,
                                  thresh_log2=math.inf, stats=stats)
    assert stats["rebases"] == 0
    assert stats["max_p"] == pytest.approx(2.0 ** 20, rel=1e-12)


def _ramp_inputs(S=512):
    """Keys whose norms grow along the sequence, so every tile raises the max."""
    q, k, v = make_random(1, 2, S, 128, seed=3001)
    ramp = torch.linspace(0.2, 6.0, S).reshape(1, 1, S, 1)
    return q, (k.float() * ramp).to(torch.bfloat16), v


CASES = {
    "normal": lambda: make_random(1, 2, 512, 128, seed=3002),
    "peaked_std2": lambda: make_random(1, 2, 512, 128, seed=3003, qk_std=2.0, v_dist="uniform"),
    "outlier_keys": lambda: make_random(1, 2, 1024, 128, seed=3004, outlier_frac=0.01),
    "ramp": _ramp_inputs,
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("block_n", [64, 128])
def test_lazy_rescale_equals_two_pass(case, block_n):
    """Skipping rescales loses nothing: the model equals the oracle to fp64 rounding."""
    q, k, v = CASES[case]()
    stats = {}
    o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_n=block_n, stats=stats)
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert (o - o_ref).abs().max().item() < 1e-12
    assert ((lse - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item() < 1e-13
    if case == "ramp":
        assert stats["rebases"] > 0
    assert stats["max_p"] <= 2.0 ** 8 * (1 + 1e-12)


@pytest.mark.parametrize("thresh", [0.0, 8.0, 15.0, 16.0, 48.0])
def test_threshold_does_not_change_result(thresh):
    q, k, v = _ramp_inputs(384)
    o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, thresh_log2=thresh)
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert (o - o_ref).abs().max().item() < 1e-12
    assert (lse - lse_ref).abs().max().item() < 1e-11


def test_bf16_p_error_is_within_budget():
    """Rounding P to bf16 before P.V (row sum unrounded) stays far inside the
    O tolerance on the peaked workload recipe."""
    q, k, v = make_random(1, 2, 512, 128, seed=3005, qk_std=2.0, v_dist="uniform")
    o, _ = online_model.online_attention(q, k, v, DEFAULT_SCALE, p_to_bf16=True)
    o_ref, _ = oracle.attention(q, k, v, DEFAULT_SCALE)
    err = (o - o_ref).abs()
    assert err.max().item() < 2e-2 / 4 and err.mean().item() < 2e-3 / 4
    assert err.max().item() > 0  # the rounding is really applied


def test_nonpositive_scale_rejected():
    q, k, v = make_random(1, 1, 128, 128, seed=3006)
    with pytest.raises(ValueError):
        online_model.online_attention(q, k, v, -1.0)


def test_rounded_rowsum_keeps_constant_v_exact():
    """Softmax weights sum to one, so O of a constant V is that constant.
    Dividing by the sum of the same bf16 P that entered P.V keeps this to
    fp64 rounding; dividing by the unrounded sum does not (it is off by the
    rounding of P, up to 2^-9 relative)."""
    q, k, _ = make_random(1, 2, 384, 128, seed=3007, qk_std=2.0)
    v = torch.full_like(q, 0.75)
    o, _ = online_model.online_attention(q, k, v, DEFAULT_SCALE, p_to_bf16=True,
                                         rowsum_of_rounded=True)
    assert (o - 0.75).abs().max().item() < 1e-14
    o_unr, _ = online_model.online_attention(q, k, v, DEFAULT_SCALE, p_to_bf16=True)
    off = (o_unr - 0.75).abs().max().item()
    assert 1e-6 < off <= 0.75 * 2.0 ** -8


def test_rounded_rowsum_error_on_outlier_recipe():
    """The 1%-outlier-key recipe with the rounded-P row sum stays inside the
    O tolerance with margin. The LSE taken from that sum differs from the
    exact one by at most -ln(1 - 2^-8) in absolute terms (each P is off by
    at most 2^-8 relative), which is within the 1e-3 relative bar wherever
    |lse| >= 3.9."""
    q, k, v = make_random(1, 2, 1024, 128, seed=3008, outlier_frac=0.01)
    o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, p_to_bf16=True,
                                           rowsum_of_rounded=True)
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    err = (o - o_ref).abs()
    assert err.max().item() < 2e-2 / 2 and err.mean().item() < 2e-3 / 2
    assert (lse - lse_ref).abs().max().item() <= -math.log1p(-2.0 ** -8)
    rel = ((lse - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item()
    assert rel < 1e-3 / 2


def test_staircase_rebases_repeatedly_at_the_kernels_thresholds():
    """The staircase key recipe of the GPU rebase tests (key norms rising
    tile by tile) makes nearly every row rebase on most tiles at the
    kernels' thresholds, 16 for the four-wave kernel (64-key tiles) and 48
    for the eight-wave kernel (128-key tiles), and at the other pairings too;
    the result still equals the two-pass oracle."""
    from workloads import staircase_keys
    q, k, v = make_random(1, 2, 1024, 128, seed=26)
    k = staircase_keys(k)
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    for block_n in (64, 128):
        for thresh in (16.0, 48.0):
            stats = {}
            o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_n=block_n,
                                                   thresh_log2=thresh, stats=stats)
            per_row = torch.cat(stats["row_rebases"])
            assert per_row.numel() == 2 * 1024
            assert (per_row >= 4).float().mean().item() >= 0.95, per_row.float().mean()
            assert per_row.float().median().item() >= 5
            assert (o - o_ref).abs().max().item() < 1e-12
            assert ((lse - lse_ref).abs() / lse_ref.abs()).max().item() < 1e-13


def test_rounded_rowsum_lse_bound_is_reached():
    """Worst case of the rounded-P row sum: with one dominant key whose
    unnormalised p is rounded to bf16, the LSE taken from that sum is off by
    close to the bound -ln(1 - 2^-8) ~= 3.9e-3 (here about 3.4e-3, above the
    1e-3 relative bar at |lse| < 1), while O stays far inside its bar."""
    q, k, v = dominant_key_small_lse_case()
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    assert 0.9 < lse_ref.item() < 0.95
    bound = -math.log1p(-2.0 ** -8)
    for block_n in (64, 128):
        o, lse = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_m=1, block_n=block_n,
                                               thresh_log2=16.0, p_to_bf16=True, rowsum_of_rounded=True)
        err = abs(lse.item() - lse_ref.item())
        assert 2.5e-3 < err <= bound
        assert (o - o_ref).abs().max().item() < 1e-3
        # the article's unrounded sum gets the LSE right in this case
        _, lse_u = online_model.online_attention(q, k, v, DEFAULT_SCALE, block_m=1, block_n=block_n,
                                                 thresh_log2=16.0, p_to_bf16=True)
        assert abs(lse_u.item() - lse_ref.item()) < 1e-12
