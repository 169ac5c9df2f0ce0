"""Helpers of the GPU tests: move generated inputs to the device and back,
and the comparison metrics. Holds none of the layer's arithmetic."""
from __future__ import annotations

import math
import sys

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None

U = 2.0 ** -24   # unit roundoff of fp32


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_available() -> bool:
    return torch is not None and torch.cuda.is_available()


def to_dev(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def to_host(t, dtype: str) -> np.ndarray:
    t = t.detach()
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class DeviceWeights:
    """Expert weights of a workload on the device (and on the host, for the
    oracle), generated once per (weight seed, shape) and reused."""
    _cache = None

    @classmethod
    def get(cls, wl):
        key = (wl.weight_seed, wl.E, wl.d, wl.d_ff, wl.dtype)
        if cls._cache is not None and cls._cache[0] == key:
            return cls._cache[1]
        cls._cache = None
        if torch is not None and torch.cuda.is_available():
            torch.cuda.empty_cache()
        host = wl.all_expert_weights()
        dev = tuple(to_dev(a, wl.dtype) for a in host)
        cls._cache = (key, (host, dev))
        return host, dev

    @classmethod
    def clear(cls):
        cls._cache = None
        if torch is not None and torch.cuda.is_available():
            torch.cuda.empty_cache()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max |got - ref| / max |ref| (the layer-output metric)."""
    got = got.reshape(got.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return np.abs(got - ref).max(axis=1) / den


def logits_tolerance(x64: np.ndarray, wr64: np.ndarray, bias) -> np.ndarray:
    """Bound for fp32 accumulation of the d products of each score: the
    products are exact (bf16 x bf16 fits fp32); each of the ~sqrt(d)-deep
    rounding levels adds at most u times the partial-sum magnitude, so
    |err| <= u (2 sqrt(d) + 8) sum_i |x_i w_i| (+ one rounding of the bias add).
    A dropped 8-element group or a wrong index exceeds this by orders of
    magnitude at the tested shapes."""
    d = x64.shape[1]
    mag = np.abs(x64) @ np.abs(wr64).T
    tol = U * (2 * math.sqrt(d) + 8) * mag
    if bias is not None:
        tol = tol + 2 * U * (mag + np.abs(np.asarray(bias, np.float64))[None, :])
    return tol + 1e-30


GUARD_WORDS = 4096   # canary elements after each guarded output


class Guarded:
    """Device outputs followed by canary regions: each array is the head of a
    larger buffer whose tail holds a fixed pattern, so a write past the end of
    an output shows up as a changed tail."""

    def __init__(self):
        self._tails = []

    def empty(self, shape, dtype, name):
        n = int(np.prod(shape)) if len(shape) else 1
        buf = torch.empty(n + GUARD_WORDS, dtype=dtype, device="cuda")
        if dtype in (torch.int32, torch.int64):
            buf.fill_(-0x5A5A5A5)
        elif dtype == torch.bfloat16:
            buf.view(torch.int16).fill_(0x5A5A)
        else:
            buf.fill_(-1234.5)
        tail = buf[n:]
        self._tails.append((name, tail, tail.clone()))
        return buf[:n].view(shape)

    def check(self):
        for name, tail, want in self._tails:
            a = tail.view(torch.int16) if tail.dtype == torch.bfloat16 else tail
            b = want.view(torch.int16) if want.dtype == torch.bfloat16 else want
            assert torch.equal(a, b), f"{name}: written past its end"
