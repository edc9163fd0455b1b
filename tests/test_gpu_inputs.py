"""The counter-based generator gives the same bits on the GPU as on the CPU
(the oracle's inputs are host copies of device-generated tensors)."""
import pytest
import torch

import moe_inputs as mi

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_generator_same_bits_on_gpu_and_cpu(dtype):
    for (seed, tag, sub, start, n) in [(0, mi.TAG_W1, 3, 0, 100000), (3, mi.TAG_X, 0, 12345, 77777),
                                       (1, mi.TAG_W2, 63, (1 << 27) - 5000, 5000)]:
        a = mi.ih4_normal(n, 0.0123, seed, tag, sub, start=start, device="cpu", out_dtype=dtype)
        b = mi.ih4_normal(n, 0.0123, seed, tag, sub, start=start, device="cuda", out_dtype=dtype)
        assert torch.equal(a.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           b.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
