"""Seeded synthetic inputs for the MoE-layer hot path.

This module feeds both sides of every parity check, the CPU oracle and the HIP
path, and holds none of the layer's arithmetic. It draws Gaussian inputs from
numpy's PCG64 with one SeedSequence per (seed, tensor, row or expert), so any
expert's weights or any token row can be regenerated on its own, in any
thread, with identical bits. bf16 tensors are returned as uint16 bit patterns
(IEEE binary32 rounded to nearest-even, top 16 bits); fp32 tensors as float32.

Near-tie rejection: a token whose top k+1 router scores have an adjacent gap
of at most 1e-3 is redrawn (stream keyed by the token and the attempt), so the
ordered top-k choice is unambiguous between an fp64 reference and an fp32
accumulation. With a rank limit M (a token may use experts of at most M of the
P ranks) the gaps are also required between the P ranks' best scores, and the
top k+1 are taken over the experts of the M ranks with the best scores. That
check is the only score this module computes, and only to accept or redraw an
input row; no result of it is ever used as an expected value.

Workloads (shapes of the models the pages use as examples):
  tiny_f32            T=64    d=128  E=8   k=2 d_ff=256   cf=1.25 fp32, seed 0
  mixtral_prefill     T=4096  d=4096 E=8   k=2 d_ff=14336 cf=1.25 bf16, seed 1
  deepseek_v3_prefill T=8192  d=7168 E=256 k=8 d_ff=2048  cf=1.25 bf16, P=8, seed 2
  zipf_skew_drops     T=16384 d=2048 E=64  k=6 d_ff=1408  cf=1.0  bf16, seed 3,
                      router bias b_e = -1.2 ln(e+1) (log of Zipf(1.2) popularity)
  deepseek_v3_decode  T=64    d=7168 E=256 k=8 d_ff=2048  cf=2.0  bf16, seed 4,
                      expert weights shared with deepseek_v3_prefill
  deepseek_v3_node_limited  as deepseek_v3_prefill with each token's experts
                      on at most M=4 of the P=8 ranks, seed 5, same weights
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GAP = 1e-3          # minimum adjacent gap among a token's top k+1 scores
MAX_ATTEMPTS = 10000

# stream ids of the tensors
_X, _WR, _WG, _WU, _WD, _DOUT = 1, 2, 3, 4, 5, 6


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest-even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a generated array."""
    if dtype == "bf16":
        return (a.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _draw(shape, std: float, dtype: str, *key: int) -> np.ndarray:
    z = _rng(*key).standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    return to_bf16_bits(z) if dtype == "bf16" else z


def host_threads() -> int:
    """Worker threads for generation: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Workload:
    """One seeded MoE-layer input set. Arrays are generated on construction,
    except the expert weights, which are drawn per expert on demand."""
    name: str
    T: int
    d: int
    E: int
    k: int
    d_ff: int
    cf: float
    dtype: str = "bf16"
    P: int = 1
    max_ranks: int = 0               # 0: no limit; else experts of at most this many ranks
    seed: int = 0
    weight_seed: int | None = None
    x_std: float = 1.0
    wr_std: float = 0.02
    bias: str | None = None          # None, "zipf1.2" or "hot0" (sends every token to expert 0)
    reject: bool = True
    x: np.ndarray = field(init=False, repr=False)
    wr: np.ndarray = field(init=False, repr=False)
    bias_vec: np.ndarray | None = field(init=False, repr=False)
    resampled: int = field(init=False, default=0)

    def __post_init__(self):
        if self.weight_seed is None:
            self.weight_seed = self.seed
        self.wr = _draw((self.E, self.d), self.wr_std, self.dtype, self.seed, _WR)
        if self.bias is None:
            self.bias_vec = None
        elif self.bias == "zipf1.2":
            self.bias_vec = (-1.2 * np.log(np.arange(1, self.E + 1, dtype=np.float64))).astype(np.float32)
        elif self.bias == "hot0":
            b = np.zeros(self.E, dtype=np.float32)
            b[0] = 1000.0
            self.bias_vec = b
        else:
            raise ValueError(f"unknown bias recipe {self.bias!r}")
        self.x = _draw((self.T, self.d), self.x_std, self.dtype, self.seed, _X)
        if self.reject and self.T > 0:
            self._reject_near_ties()

    # ---- token rows -------------------------------------------------------
    def _near_tied(self, rows: np.ndarray) -> np.ndarray:
        s = bits_to_f64(self.x[rows], self.dtype) @ bits_to_f64(self.wr, self.dtype).T
        if self.bias_vec is not None:
            s += self.bias_vec.astype(np.float64)[None, :]
        bad = np.zeros(rows.size, dtype=bool)
        if 0 < self.max_ranks < self.P:
            per = self.E // self.P
            best = s.reshape(rows.size, self.P, per).max(axis=2)
            rb = -np.sort(-best, axis=1)
            bad |= (rb[:, :-1] - rb[:, 1:]).min(axis=1) <= GAP
            keep = np.argsort(-best, axis=1, kind="stable")[:, :self.max_ranks]
            allowed = np.zeros_like(best, dtype=bool)
            np.put_along_axis(allowed, keep, True, axis=1)
            s = np.where(np.repeat(allowed, per, axis=1), s, -np.inf)
            m = min(self.k + 1, self.max_ranks * per)
        else:
            m = min(self.k + 1, self.E)
        if m < 2:
            return bad
        top = -np.sort(-s, axis=1)[:, :m]
        return bad | ((top[:, :-1] - top[:, 1:]).min(axis=1) <= GAP)

    def _reject_near_ties(self):
        bad = np.nonzero(self._near_tied(np.arange(self.T)))[0]
        attempt = 0
        while bad.size:
            attempt += 1
            if attempt > MAX_ATTEMPTS:
                raise RuntimeError("near-tie rejection did not converge")
            for t in bad:
                self.x[t] = _draw((self.d,), self.x_std, self.dtype, self.seed, _X, int(t), attempt)
            self.resampled += bad.size
            bad = bad[self._near_tied(bad)]

    # ---- upstream gradient ------------------------------------------------
    def grad_out(self, seed: int = 0) -> np.ndarray:
        """dLoss/dout [T, d] for backward checks: N(0, 1) in the layer dtype."""
        return _draw((self.T, self.d), 1.0, self.dtype, self.seed, _DOUT, seed)

    # ---- expert weights ---------------------------------------------------
    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    def expert(self, e: int):
        """(Wg [d_ff, d], Wu [d_ff, d], Wd [d, d_ff]) of expert e."""
        s, d, f = self.weight_seed, self.d, self.d_ff
        return (_draw((f, d), 1.0 / math.sqrt(d), self.dtype, s, _WG, e),
                _draw((f, d), 1.0 / math.sqrt(d), self.dtype, s, _WU, e),
                _draw((d, f), 1.0 / math.sqrt(f), self.dtype, s, _WD, e))

    def expert_chunks(self, chunk: int = 8, threads: int | None = None):
        """Yield (e0, e1, Wg, Wu, Wd) with the weights of experts [e0, e1)."""
        threads = threads or host_threads()
        with ThreadPoolExecutor(threads) as pool:
            for e0 in range(0, self.E, chunk):
                e1 = min(self.E, e0 + chunk)
                parts = list(pool.map(self.expert, range(e0, e1)))
                yield (e0, e1, np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                       np.stack([p[2] for p in parts]))

    def all_expert_weights(self, threads: int | None = None):
        """All experts at once: Wg, Wu [E, d_ff, d] and Wd [E, d, d_ff]."""
        wg = np.empty((self.E, self.d_ff, self.d), self.np_dtype)
        wu = np.empty_like(wg)
        wd = np.empty((self.E, self.d, self.d_ff), self.np_dtype)
        for e0, e1, a, b, c in self.expert_chunks(max(1, host_threads()), threads):
            wg[e0:e1], wu[e0:e1], wd[e0:e1] = a, b, c
        return wg, wu, wd


WORKLOADS = {
    "tiny_f32": dict(T=64, d=128, E=8, k=2, d_ff=256, cf=1.25, dtype="f32", seed=0,
                     x_std=1 / math.sqrt(128), wr_std=1 / math.sqrt(128)),
    "mixtral_prefill": dict(T=4096, d=4096, E=8, k=2, d_ff=14336, cf=1.25, seed=1),
    "deepseek_v3_prefill": dict(T=8192, d=7168, E=256, k=8, d_ff=2048, cf=1.25, P=8, seed=2),
    "zipf_skew_drops": dict(T=16384, d=2048, E=64, k=6, d_ff=1408, cf=1.0, seed=3, bias="zipf1.2"),
    "deepseek_v3_decode": dict(T=64, d=7168, E=256, k=8, d_ff=2048, cf=2.0, seed=4, weight_seed=2),
    "deepseek_v3_node_limited": dict(T=8192, d=7168, E=256, k=8, d_ff=2048, cf=1.25, P=8, max_ranks=4, seed=5,
                                     weight_seed=2),
}


def workload(name: str, **override) -> Workload:
    """One of the named workloads (optionally with fields overridden)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    return Workload(name=name, **cfg)


def custom(name="custom", **kw) -> Workload:
    return Workload(name=name, **kw)
