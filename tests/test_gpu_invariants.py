"""Invariants of the softmax-attention definition, run on the HIP path in
every kernel variant ("B200 attention kernel from scratch to ~SOTA in 60
figures", Chapter 1 section B: softmax does not change when a constant is
added to all of a row's scores, which is what lets the online softmax move
its base).

  * key shift: adding one vector u to every key adds sigma q_i.u to every
    score of row i, so O is unchanged and lse_i moves by sigma q_i.u;
  * joint permutation of the key and value rows: O and lse are unchanged
    (the kernel then meets the keys in another order, so its rebase
    decisions and rounding differ);
  * affine map of V: V A + 1 b^T gives O A + 1 b^T (O is a convex
    combination of the value rows).

The inputs are chosen so the transformed tensors are exact in bf16 (small
multiples of 1/8, A a signed column permutation times 1/2), so the
transformed problem is exactly the one the identity speaks of. Each output
is also compared with the oracle on its own inputs."""
import sys

import pytest
import torch

import oracle
from workloads import DEFAULT_SCALE

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_REL = 2e-2, 2e-3, 1e-3
VARIANTS = [1, 2, 3, 4]  # TILE128, PAIR256, PAIR256_EXP2EMU, PAIR128


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


def _grid(shape, gen, lo, hi):
    """Multiples of 1/8 in [lo, hi]: exact in bf16, and so are their small sums."""
    n = torch.randint(int(lo * 8), int(hi * 8) + 1, shape, generator=gen)
    return (n.to(torch.float32) / 8).to(torch.bfloat16)


def _inputs(seed, B=1, H=2, S=640):
    gen = torch.Generator().manual_seed(seed)
    shape = (B, H, S, 128)
    q = _grid(shape, gen, -1.0, 1.0)
    k = _grid(shape, gen, -2.0, 2.0)
    v = _grid(shape, gen, -4.0, 4.0)
    return q, k, v


def _run(daf, q, k, v, variant):
    dev = torch.device("cuda", 0)
    o, lse = daf.forward(q.to(dev), k.to(dev), v.to(dev), DEFAULT_SCALE, variant=variant)
    torch.cuda.synchronize()
    return o.cpu().double(), lse.cpu().double()


def _parity(o, lse, q, k, v, what):
    o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
    e = (o - o_ref).abs()
    rel = ((lse - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item()
    _say(f"{what}: O max-abs {e.max().item():.3e} mean-abs {e.mean().item():.3e} LSE max-rel {rel:.3e}")
    assert e.max().item() <= O_MAX and e.mean().item() <= O_MEAN and rel <= LSE_REL, what


@pytest.mark.parametrize("variant", VARIANTS)
def test_key_shift(daf, variant):
    _say(f"case invariant key shift variant={variant}")
    q, k, v = _inputs(501)
    gen = torch.Generator().manual_seed(502)
    u = _grid((128,), gen, -2.0, 2.0).float()
    k2 = (k.float() + u).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + u), "the shifted keys must be exact in bf16"
    o1, l1 = _run(daf, q, k, v, variant)
    o2, l2 = _run(daf, q, k2, v, variant)
    _parity(o1, l1, q, k, v, f"key shift base v{variant}")
    _parity(o2, l2, q, k2, v, f"key shift shifted v{variant}")
    d = (o2 - o1).abs()
    assert d.max().item() <= O_MAX and d.mean().item() <= O_MEAN
    shift = oracle.sigma_of(DEFAULT_SCALE) * (q.double() @ u.double())  # sigma q_i.u, per row
    assert shift.abs().max().item() > 1.0  # the shift is not negligible
    tol = 2 * LSE_REL * torch.maximum(l1.abs(), l2.abs()).clamp_min(1.0)
    assert ((l2 - l1 - shift).abs() <= tol).all()


@pytest.mark.parametrize("variant", VARIANTS)
def test_joint_key_value_permutation(daf, variant):
    _say(f"case invariant key/value permutation variant={variant}")
    q, k, v = _inputs(503)
    perm = torch.randperm(k.shape[2], generator=torch.Generator().manual_seed(504))
    k2, v2 = k[:, :, perm].contiguous(), v[:, :, perm].contiguous()
    o1, l1 = _run(daf, q, k, v, variant)
    o2, l2 = _run(daf, q, k2, v2, variant)
    _parity(o2, l2, q, k2, v2, f"permuted v{variant}")
    d = (o2 - o1).abs()
    assert d.max().item() <= O_MAX and d.mean().item() <= O_MEAN
    assert ((l2 - l1).abs() / l1.abs().clamp_min(1.0)).max().item() <= LSE_REL


@pytest.mark.parametrize("variant", VARIANTS)
def test_affine_values(daf, variant):
    _say(f"case invariant affine V variant={variant}")
    q, k, v = _inputs(505)
    gen = torch.Generator().manual_seed(506)
    cols = torch.randperm(128, generator=gen)
    signs = torch.where(torch.rand(128, generator=gen) < 0.5, -0.5, 0.5)
    A = torch.zeros((128, 128))
    A[cols, torch.arange(128)] = signs  # a signed column permutation times 1/2
    b = _grid((128,), gen, -1.0, 1.0).float()
    v2 = (v.float() @ A + b).to(torch.bfloat16)
    assert torch.equal(v2.float(), v.float() @ A + b), "the mapped values must be exact in bf16"
    o1, l1 = _run(daf, q, k, v, variant)
    o2, l2 = _run(daf, q, k, v2, variant)
    _parity(o2, l2, q, k, v2, f"affine V v{variant}")
    want = o1 @ A.double() + b.double()
    d = (o2 - want).abs()
    assert d.max().item() <= O_MAX and d.mean().item() <= O_MEAN
    assert torch.equal(l2, l1)  # the scores did not change, and the kernel is deterministic


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("e", [-64, 90])
def test_value_scale_range(daf, variant, e):
    """O is linear in V: scaling V by 2^e (exact in bf16) scales O by 2^e.
    At 2^-64 the smallest nonzero value is 2^-67, above the 2^-79 from which
    the raised base of the PAIR variants (largest p of a row down to 2^-47)
    would push p * v below fp32's normal range; at 2^90 the largest is
    2^92, where the TILE128 kernel's p of up to 2^16 summed over 640 keys
    still fits fp32. Both keep O's relative accuracy."""
    _say(f"case invariant V scale 2^{e} variant={variant}")
    q, k, v = _inputs(507)
    v2 = (v.float() * 2.0 ** e).to(torch.bfloat16)
    assert torch.equal(v2.float(), v.float() * 2.0 ** e)
    o1, l1 = _run(daf, q, k, v, variant)
    o2, l2 = _run(daf, q, k, v2, variant)
    _parity(o2 * 2.0 ** -e, l2, q, k, v, f"V scale 2^{e} v{variant}")
    d = (o2 * 2.0 ** -e - o1).abs()
    assert d.max().item() <= O_MAX and d.mean().item() <= O_MEAN
    assert torch.equal(l2, l1)  # the scores did not change
