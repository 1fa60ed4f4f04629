"""The Python binding refuses tensors the kernels cannot take (host memory, wrong dtype, rank or
shape) with ValueError before it reaches the library; no GPU is needed for these."""
import pytest
import torch

from zero_shot_rope_amd import bifocal as Z

KW = dict(w0=16, w_pretrained=64, rope_theta=1e4)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("call", [
    lambda: Z.prefill(bf16(1, 64, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), **KW),
    lambda: Z.prefill_chunk(bf16(1, 8, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), q_offset=56, **KW),
    lambda: Z.decode(bf16(1, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), L=64, **KW),
    lambda: Z.decode_step(bf16(1, 4, 128), bf16(1, 2, 128), bf16(1, 2, 128), bf16(1, 64, 2, 128),
                          bf16(1, 64, 2, 128), L=64, **KW),
    lambda: Z.decode_varlen(bf16(1, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128),
                            torch.tensor([64], dtype=torch.int32), max_len=64, **KW),
    lambda: Z.prefill_unfused(bf16(1, 64, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), **KW),
    lambda: Z.decode_unfused(bf16(1, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), L=64, **KW),
])
def test_host_tensors_are_refused(call):
    with pytest.raises(ValueError, match="CUDA/HIP"):
        call()


def test_float32_inputs_are_refused():
    with pytest.raises(ValueError, match="bfloat16"):
        Z.prefill(torch.zeros(1, 64, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), **KW)
    with pytest.raises(ValueError, match="bfloat16"):
        Z.decode(torch.zeros(1, 4, 128), bf16(1, 64, 2, 128), bf16(1, 64, 2, 128), L=64, **KW)
