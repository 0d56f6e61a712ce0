"""Shared helpers for the GPU parity tests (no arithmetic of the method)."""
import numpy as np
import torch

import oracle
import synthetic

# Parity bar: max |got - ref| / RMS(ref) over the tensor of one call.
TOL = {"bf16": 2e-2, "f32": 1e-4}

DEV = "cuda"


def dev(x):
    return None if x is None else x.to(DEV)


def f64(x):
    return synthetic.to_f64(x)


def err(got, ref):
    """RMS-normalised max error of a GPU tensor against an oracle array."""
    return oracle.rms_normalised_max_error(f64(got), ref)


def say(*a):
    print(*a, flush=True)


def out_dtype_for(dtype):
    """Parity is measured on f32 results; bf16 inputs produce f32 outputs."""
    return torch.float32


def assert_bf16_is_rounded_f32(o_bf16, o_f32):
    """A bf16 output must be exactly the f32 result rounded once."""
    assert o_bf16.dtype == torch.bfloat16 and o_f32.dtype == torch.float32
    assert torch.equal(o_f32.to(torch.bfloat16), o_bf16)
