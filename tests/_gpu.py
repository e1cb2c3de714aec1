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


def bench_lib():
    """The benchmark's measurement kernels (libexl3_bench.so), for tests that
    look at one instruction with nothing around it."""
    import ctypes
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gemm_exl3_linear_amd",
                        "libexl3_bench.so")
    L = ctypes.CDLL(path)
    L.exl3_bench_mfma_negation.restype = ctypes.c_int
    L.exl3_bench_mfma_negation.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    return L


def f16_bits(t):
    return t.detach().cpu().numpy().view(np.uint16)


def f32_bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


# ---------------------------------------------------------------------------
# full-size oracle results in reasonable time: the oracle's own functions,
# applied to independent pieces (tiles of the trellis, rows of x, expert
# tensors) in threads; numpy's array arithmetic runs outside the GIL
# ---------------------------------------------------------------------------
_WORKERS = 8


def _pool():
    import concurrent.futures as cf
    return cf.ThreadPoolExecutor(_WORKERS)


def decode_par(trellis, bits, int8=False):
    """O.decode_tensor (or decode_tensor_int8) of a whole tensor, by k-tile
    slices (tiles decode independently; the slices stack along k)."""
    fn = O.decode_tensor_int8 if int8 else O.decode_tensor
    kt = trellis.shape[0]
    cuts = np.linspace(0, kt, min(kt, 4 * _WORKERS) + 1).astype(int)
    with _pool() as ex:
        parts = list(ex.map(lambda i: fn(trellis[cuts[i]:cuts[i + 1]], bits), range(len(cuts) - 1)))
    return np.concatenate(parts, axis=0)


def rows_par(fn, x, chunk=256):
    """fn(x[rows]) over chunks of rows (the layer is row-wise), stacked."""
    import threadpoolctl
    cuts = list(range(0, x.shape[0], chunk)) + [x.shape[0]]
    with threadpoolctl.threadpool_limits(2):
        with _pool() as ex:
            parts = list(ex.map(lambda i: fn(x[cuts[i]:cuts[i + 1]]), range(len(cuts) - 1)))
    return np.concatenate(parts, axis=0)


def linear_ref(d, x=None, W=None, bias=None):
    """O.linear over all rows of x (default d["x"])."""
    x = d["x"] if x is None else x
    W = decode_par(d["trellis"], d["bits"]) if W is None else W
    return rows_par(lambda xs: O.linear(xs, d["trellis"], d["suh"], d["svh"], d["bits"], bias=bias,
                                        w_decoded=W), x)


def linear_int8_ref(d, x=None, Wq=None):
    x = d["x"] if x is None else x
    Wq = decode_par(d["trellis"], d["bits"], int8=True) if Wq is None else Wq
    return rows_par(lambda xs: O.linear_int8(xs, d["trellis"], d["suh"], d["svh"], d["bits"], wq=Wq), x)


def grouped_ref(m, tokens=None):
    """O.grouped_experts for the given tokens (all by default), with the
    expert tensors those tokens reach decoded in threads first."""
    x, ids, w = m["x"], m["ids"], m["weights"]
    if tokens is not None:
        x, ids, w = x[tokens], ids[tokens], w[tokens]
    used = sorted(set(np.unique(ids).tolist()))
    jobs = [("gate_up", e, s) for e in used for s in (0, 1)] + [("down", e, 0) for e in used]

    def width(arena, e):
        b = arena["bits"]
        return int(b[e]) if np.ndim(b) else int(b)

    def dec(job):
        kind, e, s = job
        arena = m[kind]
        return O.decode_tensor(arena["trellis"][e][s], width(arena, e))
    with _pool() as ex:
        decoded = dict(zip(jobs, ex.map(dec, jobs)))
    return O.grouped_experts(x, ids, w, m["gate_up"], m["down"], decoded=decoded)


def assert_parity(y, ref, tol=2e-3, rel_rms=5e-3, ulps=1.0, what=""):
    """Relative Frobenius error below tol over the whole array, and every
    element within rel_rms * rms(ref) + ulps fp16 ulps of its reference."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = O.rel_frobenius(y, ref)
    assert err < tol, f"{what} relative Frobenius error {err:.3e} >= {tol}"
    ex = O.elementwise_excess(y, ref, rel_rms, ulps)
    if ex > 1.0:
        bad = np.unravel_index(np.argmax(np.abs(y - ref) / (rel_rms * np.sqrt(np.mean(ref * ref))
                                                          + ulps * O.fp16_ulp(ref))), y.shape)
        raise AssertionError(f"{what} element {bad}: {y[bad]!r} against {ref[bad]!r} "
                             f"({ex:.2f} x the per-element bound)")
    return err
