"""Large shapes through the C ABI: element offsets beyond 2^31 (64-bit index
math) and a long sequence (512 K/V tiles per row), in both kernel layouts.
The oracle checks sampled rows; properties are checked over every output.
Inputs are drawn on the device with a seeded generator (16+ GiB would take
minutes to draw on the host); only the sampled heads are copied back."""
import sys

import pytest
import torch

import oracle
from workloads import DEFAULT_SCALE

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_REL = 2e-2, 2e-3, 1e-3


@pytest.fixture(scope="module")
def daf():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dense_attention_forward_amd as m
    m.lib()
    return m


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(B, H, S, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    shape = (B, H, S, 128)
    return tuple(torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                 for _ in range(3))


def _check_rows(q, k, v, o, lse, heads, rows):
    """Compare the listed (b, h) heads on the listed rows with the oracle."""
    for b, h in heads:
        qh, kh, vh = (t[b:b + 1, h:h + 1].cpu() for t in (q, k, v))
        picks = [(0, 0, r) for r in rows]
        o_ref, lse_ref = oracle.attention_rows(qh, kh, vh, DEFAULT_SCALE, picks)
        idx = torch.tensor(rows)
        og = o[b, h, idx].cpu().double()
        lg = lse[b, h, idx].cpu().double()
        e = (og - o_ref).abs()
        rel = ((lg - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item()
        _say(f"  head ({b}, {h}): O max-abs {e.max().item():.3e} mean-abs {e.mean().item():.3e} "
             f"LSE max-rel {rel:.3e}")
        assert e.max().item() <= O_MAX and e.mean().item() <= O_MEAN and rel <= LSE_REL


@pytest.mark.parametrize("variant", [1, 2, 4])
def test_offsets_beyond_int32(daf, variant):
    """B*H*S*D = 2.15e9 elements: byte offsets of the last heads exceed 2^32."""
    B, H, S = 2, 65600, 128
    _say(f"case offsets beyond 2^31 elements B={B} H={H} S={S} variant={variant}")
    q, k, v = _inputs(B, H, S, seed=41)
    assert q.numel() > 2 ** 31
    o, lse = daf.forward(q, k, v, DEFAULT_SCALE, variant=variant)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    assert (lse > 0).all().item()
    heads = [(0, 0), (0, H - 1), (1, 0), (1, H // 2), (1, H - 1)]
    _check_rows(q, k, v, o, lse, heads, [0, 1, 63, 64, 126, 127])
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", [0, 1, 2, 4])
def test_long_sequence(daf, variant):
    """S = 65536: 512 K/V tiles per row, 256 query-tile pairs per head."""
    B, H, S = 1, 2, 65536
    _say(f"case long sequence B={B} H={H} S={S} variant={variant} (library pick "
         f"{daf.pick(B, H, S)})")
    q, k, v = _inputs(B, H, S, seed=42)
    o, lse = daf.forward(q, k, v, DEFAULT_SCALE, variant=variant)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    vmin = v.float().amin(dim=2, keepdim=True)
    vmax = v.float().amax(dim=2, keepdim=True)
    of = o.float()
    assert ((of >= vmin - O_MAX) & (of <= vmax + O_MAX)).all().item()
    _check_rows(q, k, v, o, lse, [(0, 0), (0, 1)], [0, 127, 128, 255, 32767, 32768, 65407, 65535])
