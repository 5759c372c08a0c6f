"""The MFMA-rate probe (include/attn_mfma_rate.h) runs through the C ABI:
its result is finite and the accumulation is linear in the iteration count
(every round adds the same products)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_mfma_rate_accumulates_linearly():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import dense_attention_forward_amd as daf
    wgs = 8
    gen = torch.Generator(device="cuda").manual_seed(3)
    operands = torch.randn(wgs * 256 * 64, generator=gen, device="cuda").to(torch.bfloat16)
    s10 = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    s20 = torch.empty_like(s10)
    assert daf.mfma_rate(operands, s10, wgs, 10) == wgs * 10 * 4 * 16 * 32768
    daf.mfma_rate(operands, s20, wgs, 20)
    torch.cuda.synchronize()
    assert torch.isfinite(s10).all() and (s10 != 0).any()
    err = (s20.double() - 2 * s10.double()).abs().max().item()
    assert err <= 1e-4 * s10.double().abs().max().item() + 1e-3
