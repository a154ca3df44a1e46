"""Seeded synthetic recurrent Q/K/V workloads (input synthesis only).

This module is shared by the tests, the benchmark and the oracle-side checks.
It holds none of the attention arithmetic: it only draws Gaussian tensors,
plants key blocks and rounds to bf16.  Every tensor is a deterministic
function of (config, seed, tensor, batch, head, step), so any head of any
step can be regenerated on its own (the oracle only needs the heads it
checks), and the full-tensor iterator yields bit-identical values.

Workload recipe (the pages run real Huginn / HotpotQA trajectories; these
synthetic inputs stand in for their shapes only):

* base tensors Q0, K0, V0 ~ N(0, 1), fp32, one independent PCG64 stream per
  (tensor, batch, head, step);
* planting: for every query block q, ``planted`` key blocks are drawn
  uniformly without replacement from {1, ..., q-1} (the sink block 0 and the
  diagonal block q are excluded because the selection always keeps them);
  each planted block's keys get ``beta * sqrt(D) * u_q`` added, where u_q is
  the unit vector along the mean of the base queries of block q.  Shifts from
  different query blocks add up.  Optionally each other off-diagonal,
  non-sink block also gets a ``random_beta`` shift with probability
  ``random_frac``;
* drift: X(t) = X(t-1) + sigma * N(0, 1) for t >= 1 (fp32 random walk);
* handoff: every step is rounded to bf16 (round-to-nearest-even) and passed as
  raw uint16 bits, identical for the GPU and for the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, Optional, Tuple

import numpy as np

__all__ = ["WorkloadConfig", "CONFIGS", "Workload", "round_to_bf16_bits",
           "bf16_bits_to_f32"]

_SEED_BASE = 20261202
_TENSOR_Q, _TENSOR_K, _TENSOR_V, _TENSOR_PLANT = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    batch: int
    heads: int
    head_dim: int
    seq_len: int
    block: int
    steps: int          # recurrent depth T
    td: int             # discovery steps (dense), steps td..T-1 are sparse
    eta: float          # cumulative-mass threshold
    cap: int            # per-row cap on eta-ranked blocks (0 = none)
    planted: Tuple[int, int]   # (lo, hi) planted blocks per query block; lo == hi is fixed
    beta: float         # planted shift, in units of sqrt(D) along u_q
    sigma: float        # per-step drift std
    random_frac: float = 0.0
    random_beta: float = 0.0
    index: int = 0      # seed offset

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def seed(self) -> int:
        return _SEED_BASE + self.index

    def with_(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


def _cfg(name, index, **kw):
    return WorkloadConfig(name=name, index=index, **kw)


# Shapes of the five workloads the method is evaluated on here (Huginn-like
# 55-head d=96 geometry, 4K-32K multi-hop contexts).
CONFIGS = {
    "tiny": _cfg("tiny", 0, batch=1, heads=4, head_dim=64, seq_len=256, block=32,
                 steps=4, td=2, eta=0.90, cap=0, planted=(3, 3), beta=1.5,
                 sigma=0.05),
    "ctx4k": _cfg("ctx4k", 1, batch=1, heads=32, head_dim=128, seq_len=4096,
                  block=64, steps=32, td=8, eta=0.90, cap=0, planted=(8, 8),
                  beta=2.0, sigma=0.02),
    "ctx8k": _cfg("ctx8k", 2, batch=1, heads=32, head_dim=128, seq_len=8192,
                  block=64, steps=32, td=8, eta=0.90, cap=0, planted=(8, 8),
                  beta=2.0, sigma=0.02),
    "ctx16k": _cfg("ctx16k", 2, batch=1, heads=32, head_dim=128, seq_len=16384,
                   block=64, steps=32, td=8, eta=0.90, cap=0, planted=(8, 8),
                   beta=2.0, sigma=0.02),
    "ctx32k": _cfg("ctx32k", 2, batch=1, heads=32, head_dim=128, seq_len=32768,
                   block=64, steps=32, td=8, eta=0.90, cap=0, planted=(8, 8),
                   beta=2.0, sigma=0.02),
    "wide": _cfg("wide", 3, batch=8, heads=55, head_dim=96, seq_len=4096,
                 block=64, steps=32, td=8, eta=0.95, cap=0, planted=(4, 16),
                 beta=2.0, sigma=0.02),
    "long": _cfg("long", 4, batch=1, heads=40, head_dim=128, seq_len=32768,
                 block=128, steps=16, td=4, eta=0.90, cap=64, planted=(12, 12),
                 beta=2.0, sigma=0.02, random_frac=0.02, random_beta=0.5),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits with round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32 (for reporting only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: WorkloadConfig, tensor: int, b: int, h: int, step: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=cfg.seed, spawn_key=(tensor, b, h, step))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(cfg, tensor, b, h, step):
    return _rng(cfg, tensor, b, h, step).standard_normal(
        (cfg.seq_len, cfg.head_dim), dtype=np.float32)


def _plant_shift(cfg: WorkloadConfig, b: int, h: int, q0: np.ndarray) -> np.ndarray:
    """Key shift of one (batch, head): sum of beta*sqrt(D)*u_q over planted (q, kb)."""
    nb, B, D = cfg.n_blocks, cfg.block, cfg.head_dim
    g = _rng(cfg, _TENSOR_PLANT, b, h, 0)
    lo, hi = cfg.planted
    count = int(g.integers(lo, hi + 1)) if hi > lo else lo
    shift_per_block = np.zeros((nb, D), dtype=np.float64)
    qmean = q0.reshape(nb, B, D).astype(np.float64).mean(axis=1)
    for q in range(nb):
        cand = np.arange(1, q, dtype=np.int64)       # excludes sink 0 and diagonal q
        take = min(count, cand.size)
        planted = g.choice(cand, size=take, replace=False) if take > 0 else cand[:0]
        norm = np.linalg.norm(qmean[q])
        u = qmean[q] / norm if norm > 0 else np.zeros(D)
        for kb in planted:
            shift_per_block[kb] += cfg.beta * math.sqrt(D) * u
        if cfg.random_frac > 0 and cand.size > 0:
            rest = np.setdiff1d(cand, planted, assume_unique=True)
            hit = rest[g.random(rest.size) < cfg.random_frac]
            for kb in hit:
                shift_per_block[kb] += cfg.random_beta * math.sqrt(D) * u
    return np.repeat(shift_per_block, B, axis=0).astype(np.float32)


class Workload:
    """Deterministic recurrent Q/K/V trajectory for one config."""

    def __init__(self, cfg: WorkloadConfig, threads: int = 8):
        self.cfg = cfg
        self.threads = max(1, threads)

    # ---- one (batch, head) -------------------------------------------------
    def head_base(self, b: int, h: int):
        cfg = self.cfg
        q0 = _normal(cfg, _TENSOR_Q, b, h, 0)
        k0 = _normal(cfg, _TENSOR_K, b, h, 0)
        v0 = _normal(cfg, _TENSOR_V, b, h, 0)
        k0 = k0 + _plant_shift(cfg, b, h, q0)
        return [q0, k0, v0]

    def _drift(self, masters, b, h, step):
        s = np.float32(self.cfg.sigma)
        for i, tensor in enumerate((_TENSOR_Q, _TENSOR_K, _TENSOR_V)):
            masters[i] = masters[i] + s * _normal(self.cfg, tensor, b, h, step)

    def head_step(self, b: int, h: int, t: int):
        """bf16 bits (q, k, v), each [S, D], of (batch b, head h) at step t."""
        masters = self.head_base(b, h)
        for step in range(1, t + 1):
            self._drift(masters, b, h, step)
        return tuple(round_to_bf16_bits(m) for m in masters)

    def head_steps(self, b: int, h: int, steps=None):
        """Iterate (t, (q, k, v) bits) over steps of one head."""
        T = self.cfg.steps if steps is None else steps
        masters = self.head_base(b, h)
        for t in range(T):
            if t > 0:
                self._drift(masters, b, h, t)
            yield t, tuple(round_to_bf16_bits(m) for m in masters)

    # ---- whole tensors --------------------------------------------------------
    def steps(self, n_steps: Optional[int] = None) -> Iterator[Tuple[int, np.ndarray, np.ndarray, np.ndarray]]:
        """Iterate (t, q, k, v) with bf16 bits shaped [batch, heads, S, D]."""
        cfg = self.cfg
        T = cfg.steps if n_steps is None else n_steps
        units = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
        shape = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
        with ThreadPoolExecutor(self.threads) as pool:
            masters = list(pool.map(lambda u: self.head_base(*u), units))
            for t in range(T):
                if t > 0:
                    list(pool.map(lambda iu: self._drift(masters[iu[0]], iu[1][0], iu[1][1], t),
                                  enumerate(units)))
                out = [np.empty(shape, dtype=np.uint16) for _ in range(3)]

                def _round(iu):
                    i, (b, h) = iu
                    for j in range(3):
                        out[j][b, h] = round_to_bf16_bits(masters[i][j])
                list(pool.map(_round, enumerate(units)))
                yield t, out[0], out[1], out[2]
