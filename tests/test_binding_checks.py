"""The Python binding rejects tensors the library cannot take before any call
into it: host tensors, wrong dtypes, shapes or layouts (CPU only)."""

import pytest
import torch

import context_attention_diffusion_ringattn_amd as ra


def test_acc_init_rejects_host_and_malformed_accumulators():
    with pytest.raises(ValueError, match="ROCm device"):
        ra.acc_init(torch.zeros(1, 4, 2, 64), torch.zeros(1, 2, 4))
    with pytest.raises(ValueError, match="ROCm device"):
        ra.acc_init(torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16), torch.zeros(1, 2, 4))
    with pytest.raises(ValueError):
        ra.acc_init(torch.zeros(4, 2, 64), torch.zeros(1, 2, 4))


def test_merge_rejects_host_tensors():
    o = torch.zeros(1, 4, 2, 64)
    l = torch.zeros(1, 2, 4)
    with pytest.raises(ValueError, match="ROCm device"):
        ra.merge(o, l, o.clone(), l.clone())


@pytest.mark.parametrize("call", ["forward", "step", "ring_sweep", "step_bf16"])
def test_attention_calls_reject_host_inputs(call):
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="ROCm device"):
        if call == "forward":
            ra.forward(q, k, k.clone(), ring_degree=2)
        elif call == "ring_sweep":
            ra.ring_sweep(k, k, k.clone(), ring_degree=2)
        elif call == "step":
            ra.step(q, k, k.clone(), torch.zeros(1, 4, 2, 64), torch.zeros(1, 2, 4))
        else:
            ra.step_bf16(q, k, k.clone(), torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16),
                         torch.zeros(1, 2, 4, dtype=torch.bfloat16))


def test_attention_calls_reject_wrong_dtype_and_layout():
    k = torch.zeros(1, 8, 2, 64, dtype=torch.float16)
    with pytest.raises(TypeError, match="bfloat16"):
        ra.forward(k, k, k, ring_degree=2)
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        ra.forward(q, q, q)
