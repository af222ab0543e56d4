"""The benchmark's model glue between decode layers (libmoebench.so, not the layer
library): x_out = bf16(x + y), n_out = bf16(x_out / sqrt(mean(x_out^2) + eps)).

Checked against the same formula in fp32 torch ops on the CPU: x_out bit for bit
(one fp32 add of two bf16 values, rounded once); n_out within one bf16 ulp, since
the fp32 sum of squares may be added up in another order (the scale 1/sqrt(.) then
differs in its last bits and can move a rounding boundary).
"""
import pytest

pytestmark = pytest.mark.gpu


def _ref(x, y, eps):
    import torch
    xs = x.float() if y is None else (x.float() + y.float()).to(torch.bfloat16).float()
    r = 1.0 / torch.sqrt((xs * xs).sum(dim=1, keepdim=True) / x.shape[1] + eps)
    return xs.to(torch.bfloat16), (xs * r).to(torch.bfloat16)


@pytest.mark.parametrize("T,H,with_y", [(1, 2048, True), (3, 4096, True), (2, 8192, False), (5, 520, True)])
def test_residual_rmsnorm_matches_formula(gpu, T, H, with_y):
    import torch
    from quantized_routed_expert_softmax_amd import benchlib

    g = torch.Generator().manual_seed(1000 + T * 7 + H)
    x = (torch.randn(T, H, generator=g) * 1.7).to(torch.bfloat16)
    y = (torch.randn(T, H, generator=g) * 0.3).to(torch.bfloat16) if with_y else None
    xd, yd = x.to(gpu), (y.to(gpu) if y is not None else None)
    x_out = torch.empty_like(xd)
    n_out = torch.empty_like(xd)
    benchlib.residual_rmsnorm(xd, yd, x_out, n_out, eps=1e-6)
    torch.cuda.synchronize()
    rx, rn = _ref(x, y, 1e-6)
    if with_y:
        assert torch.equal(x_out.cpu(), rx)
    got = n_out.cpu().float()
    ulp = torch.ldexp(torch.ones_like(got), torch.frexp(rn.float().abs().clamp_min(1e-30))[1] - 8)
    assert bool(((got - rn.float()).abs() <= ulp).all()), float((got - rn.float()).abs().max())


def test_residual_rmsnorm_refuses_too_wide_rows(gpu):
    import torch
    from quantized_routed_expert_softmax_amd import benchlib

    x = torch.zeros(1, 64 * 8 * 16 + 8, dtype=torch.bfloat16, device=gpu)
    with pytest.raises(RuntimeError):
        benchlib.residual_rmsnorm(x, None, torch.empty_like(x), torch.empty_like(x))
