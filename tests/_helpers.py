"""Shared helpers of the GPU parity tests (inputs, tolerances, oracle cache)."""

import functools

import numpy as np
import pytest
import torch

from fp8_transformer_step_amd import inputs

# Tolerances (max relative error = max|gpu - ref| / max|ref|).
TOL_FP8_PATH = 2e-2
TOL_BF16_ATTN = 5e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def max_rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def to_dev_bf16(bits):
    """uint16 bf16 bits (NumPy) -> bf16 CUDA tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def from_dev_bf16(t):
    """bf16 CUDA tensor -> float64 NumPy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def f32(bits):
    return inputs.bf16_bits_to_f32(bits)


@functools.lru_cache(maxsize=4)
def mlp_weights_cached(workload, hidden, inter):
    return inputs.mlp_weights(workload, hidden, inter)


def log(msg):
    print(msg, flush=True)
