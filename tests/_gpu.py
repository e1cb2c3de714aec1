"""Helpers for the GPU parity tests: device copies of synthetic inputs and
cached oracle results (the oracle runs on the host, the library on cuda:0)."""
import functools

import numpy as np

import synth
from oracle import exl3_oracle as O


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def weight(d, bias=None):
    import gemm_exl3_linear_amd as X
    return X.Exl3Weight.from_numpy(d["trellis"], d["suh"], d["svh"], d["bits"], bias=bias, device=dev())


@functools.lru_cache(maxsize=8)
def linear_case(seed, m, k, n, bits):
    d = synth.linear_inputs(seed, m, k, n, bits)
    return d


@functools.lru_cache(maxsize=8)
def decoded(seed, m, k, n, bits):
    d = linear_case(seed, m, k, n, bits)
    return O.decode_tensor(d["trellis"], bits)


def f16_bits(t):
    return t.detach().cpu().numpy().view(np.uint16)
