"""Seeded synthetic sampler inputs, shared by the oracle tests, the GPU parity tests and the bench.

This module only draws numbers: logits matrices and per-row sampling parameters. It holds no
step of the sampling method itself (no softmax, no filtering, no random race), so both the CPU
oracle and the HIP path can consume its output without sharing any of the method's arithmetic.

The six workloads follow the shapes and value distributions of the sampling-mask pages: a
decode batch of logits rows over an LLM vocabulary, per-row temperature / top-k / top-p / min-p,
a subset of rows that opt in to support capture, and per-request seeds.
Real model logits are not available, so Gaussian logits (optionally plus a log-Zipf rank bonus,
which gives the heavy head a language model's next-token distribution has) stand in for them.

Recipe (each workload draws from ``numpy.random.default_rng(index - 1)`` in this order):
  1. logits, row by row: ``standard_normal(V) * sigma``; for Zipf workloads then
     ``permutation(V) + 1`` as the rank of each token, and the bonus ``a * ln(rank**-s / H(V, s))``
     with ``H`` the generalized harmonic number; the 0.125-grid workload rounds to that grid;
     fp32 workloads cast to float32, bf16 workloads cast to float32 and then round to nearest
     even bfloat16 (stored as the raw uint16 bit patterns);
  2. per-row parameters (only those that vary), in the order temperature, top_k, top_p, min_p,
     greedy rows, opt-in rows.
Seeds are ``1_000_003 * index + row`` and positions are 0 for every row.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = ["Workload", "make_workload", "WORKLOADS", "f32_to_bf16_bits", "bf16_bits_to_f32"]


@dataclasses.dataclass
class Workload:
    """One batch of sampler inputs.

    ``logits`` is ``float32 [B, V]`` for dtype ``"f32"`` and ``uint16 [B, V]`` (raw bfloat16 bit
    patterns) for dtype ``"bf16"``. Parameter arrays are ``[B]``; ``optin_rows`` is strictly
    ascending int32; ``W`` is the packed width of the capture outputs.
    """

    name: str
    dtype: str
    logits: np.ndarray
    temperature: np.ndarray  # float32 [B]
    top_k: np.ndarray  # int32 [B]
    top_p: np.ndarray  # float32 [B]
    min_p: np.ndarray  # float32 [B]
    optin_rows: np.ndarray  # int32 [R]
    seeds: np.ndarray  # uint64 [B]
    positions: np.ndarray  # uint64 [B]
    W: int

    @property
    def B(self) -> int:
        return int(self.logits.shape[0])

    @property
    def V(self) -> int:
        return int(self.logits.shape[1])

    @property
    def R(self) -> int:
        return int(self.optin_rows.shape[0])

    def digest(self) -> str:
        """SHA-256 over every input array, in a fixed order."""
        h = hashlib.sha256()
        for a in (self.logits, self.temperature, self.top_k, self.top_p, self.min_p,
                  self.optin_rows, self.seeds, self.positions):
            h.update(np.ascontiguousarray(a).tobytes())
        h.update(str(self.W).encode())
        return h.hexdigest()

    def rows(self, idx) -> "Workload":
        """A workload holding only rows ``idx`` (opt-in rows re-indexed to the subset)."""
        idx = np.asarray(idx, dtype=np.int64)
        opt = set(int(r) for r in self.optin_rows)
        new_opt = np.array([j for j, r in enumerate(idx) if int(r) in opt], dtype=np.int32)
        return dataclasses.replace(
            self, name=f"{self.name}[rows]", logits=np.ascontiguousarray(self.logits[idx]),
            temperature=self.temperature[idx].copy(), top_k=self.top_k[idx].copy(),
            top_p=self.top_p[idx].copy(), min_p=self.min_p[idx].copy(), optin_rows=new_opt,
            seeds=self.seeds[idx].copy(), positions=self.positions[idx].copy())


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns uint16 bit patterns.

    Inputs must be finite (the generator never produces NaN)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def perturbed_logits(logits: np.ndarray, dtype: str, seed: int, sigma: float = 0.25) -> np.ndarray:
    """New logits for a replay: the given [B, V] logits (float32, or uint16 bfloat16 bits) plus
    seeded N(0, sigma^2) noise, rounded back to the same dtype; -inf entries stay -inf. Stands
    in for a training model's logits at the captured positions, a small step away from the
    sampling model's."""
    rng = np.random.default_rng(seed)
    x = bf16_bits_to_f32(logits) if dtype == "bf16" else np.asarray(logits, np.float32)
    noise = (rng.standard_normal(x.shape) * sigma).astype(np.float32)
    finite = np.isfinite(x)
    y = np.where(finite, x + noise, x).astype(np.float32)
    if dtype != "bf16":
        return y
    out = f32_to_bf16_bits(np.where(finite, y, 0.0))
    out[~finite] = np.asarray(logits)[~finite]
    return out


def _zipf_bonus(rng: np.random.Generator, V: int, s: float, a: float) -> np.ndarray:
    rank = rng.permutation(V).astype(np.float64) + 1.0
    H = np.sum(np.arange(1, V + 1, dtype=np.float64) ** (-s))
    return a * (-s * np.log(rank) - np.log(H))


def _logits(rng, B, V, sigma, dtype, zipf=None, grid=None) -> np.ndarray:
    out = np.empty((B, V), dtype=np.float32 if dtype == "f32" else np.uint16)
    for r in range(B):
        x = rng.standard_normal(V) * sigma
        if zipf is not None:
            x = x + _zipf_bonus(rng, V, *zipf)
        if grid is not None:
            x = np.round(x / grid) * grid
        x32 = x.astype(np.float32)
        out[r] = x32 if dtype == "f32" else f32_to_bf16_bits(x32)
    return out


def _seeds(index: int, B: int) -> np.ndarray:
    return (np.uint64(1_000_003) * np.uint64(index) + np.arange(B, dtype=np.uint64)).astype(np.uint64)


def _full(B, v, dt):
    return np.full(B, v, dtype=dt)


def make_workload(index: int, *, W: Optional[int] = None) -> Workload:
    """Build workload ``index`` (1..6). ``W`` overrides the packed width."""
    rng = np.random.default_rng(index - 1)
    if index == 1:
        B, V = 4, 1024
        x = _logits(rng, B, V, 2.0, "f32")
        wl = Workload("b4_v1024_f32", "f32", x, _full(B, 1.0, np.float32), _full(B, 8, np.int32),
                      _full(B, 0.9, np.float32), _full(B, 0.0, np.float32),
                      np.arange(B, dtype=np.int32), _seeds(index, B), np.zeros(B, np.uint64), 16)
    elif index == 2:
        B, V = 64, 32000
        x = _logits(rng, B, V, 1.0, "f32", zipf=(1.1, 3.0))
        wl = Workload("b64_v32000_f32_zipf", "f32", x, _full(B, 1.0, np.float32),
                      _full(B, 50, np.int32), _full(B, 0.95, np.float32), _full(B, 0.0, np.float32),
                      np.arange(0, B, 2, dtype=np.int32), _seeds(index, B), np.zeros(B, np.uint64), 64)
    elif index == 3:
        B, V = 256, 151936
        x = _logits(rng, B, V, 2.5, "bf16", grid=0.125)
        T = rng.uniform(0.6, 1.2, B).astype(np.float32)
        wl = Workload("b256_v151936_bf16_grid", "bf16", x, T, _full(B, 1024, np.int32),
                      _full(B, 0.95, np.float32), _full(B, 0.0, np.float32),
                      np.arange(B, dtype=np.int32), _seeds(index, B), np.zeros(B, np.uint64), 2048)
    elif index == 4:
        B, V = 256, 129280
        x = _logits(rng, B, V, 1.5, "bf16")
        wl = Workload("b256_v129280_bf16_k8192", "bf16", x, _full(B, 1.0, np.float32),
                      _full(B, 8192, np.int32), _full(B, 1.0, np.float32), _full(B, 0.0, np.float32),
                      np.arange(B, dtype=np.int32), _seeds(index, B), np.zeros(B, np.uint64), 8192)
    elif index == 5:
        B, V = 1024, 262144
        x = _logits(rng, B, V, 1.0, "bf16", zipf=(1.2, 4.0))
        T = rng.uniform(0.5, 1.5, B).astype(np.float32)
        k = rng.integers(1, 4097, B).astype(np.int32)
        p = rng.uniform(0.8, 1.0, B).astype(np.float32)
        mp = rng.uniform(0.0, 0.1, B).astype(np.float32)
        greedy = rng.choice(B, 102, replace=False)
        T[greedy] = 0.0
        opt = np.sort(rng.choice(B, 256, replace=False)).astype(np.int32)
        wl = Workload("b1024_v262144_bf16_mixed", "bf16", x, T, k, p, mp, opt,
                      _seeds(index, B), np.zeros(B, np.uint64), 4608)
    elif index == 6:
        # The mixed batch's logits recipe with top-k off on every row: pure top-p (U[0.8, 1.0]),
        # min-p U[0, 0.1] on half the rows, temperature U[0.5, 1.5], 25% of rows opt-in.
        B, V = 1024, 262144
        x = _logits(rng, B, V, 1.0, "bf16", zipf=(1.2, 4.0))
        T = rng.uniform(0.5, 1.5, B).astype(np.float32)
        p = rng.uniform(0.8, 1.0, B).astype(np.float32)
        mp = rng.uniform(0.0, 0.1, B).astype(np.float32)
        mp[rng.choice(B, B // 2, replace=False)] = 0.0
        opt = np.sort(rng.choice(B, 256, replace=False)).astype(np.int32)
        wl = Workload("b1024_v262144_bf16_topk_off", "bf16", x, T, _full(B, -1, np.int32), p, mp,
                      opt, _seeds(index, B), np.zeros(B, np.uint64), 4608)
    else:
        raise ValueError(f"unknown workload {index}")
    if W is not None:
        wl.W = int(W)
    return wl


WORKLOADS = {1: "b4_v1024_f32", 2: "b64_v32000_f32_zipf", 3: "b256_v151936_bf16_grid",
             4: "b256_v129280_bf16_k8192", 5: "b1024_v262144_bf16_mixed",
             6: "b1024_v262144_bf16_topk_off"}
