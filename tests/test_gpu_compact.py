"""GPU parity of the compact 3-bit activation codes (MX_UE2M1) used for the
latent-replay buffer (MicroQonv, arXiv 2609.28358, §VI-A: the sign bit of
post-ReLU activations removed, 3.125 bits per element with the block scale;
§VII).  Codes (packed 3-bit stream), block scales, T and amax bit-exact
against the oracle; dequantization bit-exact; and for post-ReLU data the
dequantized values equal those of the 4-bit E2M1 codes."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mx_amd as mx
import oracle as O
from microscaling_quantized_convolution_mx_amd import workloads as WL
from gpu_util import DEV, f32_bits, gpu_quantize, say

pytestmark = pytest.mark.gpu

SHAPES = [  # (n, c, h, w): ragged group counts, one block, the full replay buffer
    (8, 8, 1, 1),
    (16, 24, 5, 3),
    (64, 64, 8, 8),
    (10000, 64, 8, 8),
]


def act_desc(n, c, h, w, fmt):
    return mx.desc(n, c, 8, h, w, 1, 1, elem_fmt=fmt)


@pytest.mark.parametrize("relu", [True, False])
@pytest.mark.parametrize("shape", SHAPES)
def test_compact_codes_bit_exact(shape, relu):
    n, c, h, w = shape
    say("compact", shape, relu)
    x = torch.randn(h, w, c, n, generator=torch.Generator().manual_seed(n + c + h))
    if relu:
        x = torch.relu(x)
    d = act_desc(n, c, h, w, mx.MX_UE2M1)
    q = gpu_quantize(d, mx.MX_ROLE_ACT, x)
    back = torch.empty(h, w, c, n, device=DEV)
    mx.mx_dequantize(d, mx.MX_ROLE_ACT, q, back)
    torch.cuda.synchronize()
    ref = O.quantize(O.ACT, O.UE2M1, x.numpy())
    assert np.array_equal(q.codes[:q.code_bytes].cpu().numpy(), ref.packed())
    assert np.array_equal(q.scales[:q.nblocks].cpu().numpy(), ref.scales)
    assert f32_bits(q.tensor_scale.item()) == f32_bits(ref.t)
    assert f32_bits(q.amax.item()) == f32_bits(ref.amax)
    assert np.array_equal(back.cpu().numpy().view(np.uint32), O.dequantize(ref).view(np.uint32))
    if relu:
        d4 = act_desc(n, c, h, w, mx.MX_E2M1)
        q4 = gpu_quantize(d4, mx.MX_ROLE_ACT, x)
        back4 = torch.empty_like(back)
        mx.mx_dequantize(d4, mx.MX_ROLE_ACT, q4, back4)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int32), back4.view(torch.int32))
        # 3 bits + 8/64 per element
        assert (q.code_bytes + q.nblocks) * 8 == 3.125 * x.numel()
