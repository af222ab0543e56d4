"""Router logits for the lookahead guesses, GPU vs the fp64 oracle.

Source: "RFC: stream MoE experts from disk in from_pretrained", How the
prototype works, Reads bullet (the next layers' routers run on the current
hidden states).  bf16 x bf16 products are exact in fp32, so the only error is
fp32 summation over H terms: |got - exact| <= H * 2^-24 * sum_i |x_i w_i|.
"""
import numpy as np
import pytest

import oracle
from quantized_routed_expert_softmax_amd import binding as B
from quantized_routed_expert_softmax_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,E,n,seed", [
    (1, 2048, 128, 3, 0),     # mixed decode: this layer and the next two
    (8, 2048, 128, 3, 1),     # batch 8: two token chunks
    (1, 2048, 512, 3, 2),     # decode workload's width
    (9, 256, 1, 8, 3),        # ragged token chunk, E = 1, most routers at once
    (5, 72, 7, 2, 4),         # H not a multiple of 512: partial lane coverage
    (33, 4096, 256, 1, 5),    # wide hidden size, many chunks
])
def test_router_logits_within_summation_bound(T, H, E, n, seed):
    import torch
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    w = synth.f32_to_bf16_bits((rng.standard_normal((n, E, H)) / np.sqrt(H)).astype(np.float32))
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    got = B.moe_router_logits(xd, wd).cpu().numpy().astype(np.float64)
    ref = oracle.router_logits(x, w)
    xf = np.abs(synth.bf16_bits_to_f32(x).astype(np.float64))
    wf = np.abs(synth.bf16_bits_to_f32(w).astype(np.float64))
    bound = np.einsum("ti,mei->mte", xf, wf) * H * 2.0 ** -24 + 1e-30
    assert got.shape == ref.shape
    assert np.all(np.abs(got - ref) <= bound)


def test_router_logits_empty_and_bad_arguments():
    import torch
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    assert B.moe_router_logits(x, w).shape == (1, 0, 4)
    with pytest.raises(B.MoeError):
        B.moe_router_logits(torch.zeros((1, 60), dtype=torch.bfloat16, device="cuda"),
                            torch.zeros((1, 4, 60), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(B.MoeError):
        B.moe_router_logits(torch.zeros((1, 64), dtype=torch.bfloat16, device="cuda"),
                            torch.zeros((9, 4, 64), dtype=torch.bfloat16, device="cuda"))
