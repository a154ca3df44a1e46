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
* grouped-query attention (``kv_heads`` < ``heads``): query head h reads
  key/value head h // (heads / kv_heads); each key head receives the planted
  shifts of every query head of its group (they add up, as above);
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
    kv_heads: int = 0   # key/value heads (0: one per query head)

    @property
    def n_blocks(self) -> int:
        return self.seq_len // self.block

    @property
    def n_kv(self) -> int:
        return self.kv_heads or self.heads

    @property
    def group(self) -> int:
        """Query heads per key/value head."""
        return self.heads // self.n_kv

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
    # The 4K inputs (same seeds) selected at eta = 0.6: the support then covers
    # about 15% of the full block grid, the density the 4K workload
    # description states; eta differs from that workload's 0.9.
    "ctx4k_eta06": _cfg("ctx4k_eta06", 1, batch=1, heads=32, head_dim=128, seq_len=4096,
                        block=64, steps=32, td=8, eta=0.60, cap=0, planted=(8, 8),
                        beta=2.0, sigma=0.02),
    # Recurrent-Llama-like grouped-query geometry: 32 query heads, 8 KV heads.
    "gqa4k": _cfg("gqa4k", 5, batch=1, heads=32, kv_heads=8, head_dim=128, seq_len=4096,
                  block=64, steps=32, td=8, eta=0.90, cap=0, planted=(8, 8),
                  beta=2.0, sigma=0.02),
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

    # ---- base tensors --------------------------------------------------------
    def q_base(self, b: int, h: int) -> np.ndarray:
        return _normal(self.cfg, _TENSOR_Q, b, h, 0)

    def kv_base(self, b: int, g: int, q0s=None):
        """[k0, v0] of key/value head g; q0s: the base queries of its query
        heads g*G .. g*G+G-1 (generated when not given)."""
        cfg = self.cfg
        G = cfg.group
        if q0s is None:
            q0s = [self.q_base(b, g * G + i) for i in range(G)]
        k0 = _normal(cfg, _TENSOR_K, b, g, 0)
        for i in range(G):
            k0 = k0 + _plant_shift(cfg, b, g * G + i, q0s[i])
        v0 = _normal(cfg, _TENSOR_V, b, g, 0)
        return [k0, v0]

    def head_base(self, b: int, h: int):
        """[q0, k0, v0] seen by query head h."""
        G = self.cfg.group
        g = h // G
        q0s = [self.q_base(b, g * G + i) for i in range(G)]
        return [q0s[h - g * G]] + self.kv_base(b, g, q0s)

    def _drift_one(self, master, tensor, b, hh, step):
        return master + np.float32(self.cfg.sigma) * _normal(self.cfg, tensor, b, hh, step)

    def head_steps(self, b: int, h: int, steps=None):
        """Iterate (t, (q, k, v) bits) over steps of one query head (k, v of
        its key/value head)."""
        cfg = self.cfg
        T = cfg.steps if steps is None else steps
        g = h // cfg.group
        q, k, v = self.head_base(b, h)
        for t in range(T):
            if t > 0:
                q = self._drift_one(q, _TENSOR_Q, b, h, t)
                k = self._drift_one(k, _TENSOR_K, b, g, t)
                v = self._drift_one(v, _TENSOR_V, b, g, t)
            yield t, tuple(round_to_bf16_bits(m) for m in (q, k, v))

    def head_step(self, b: int, h: int, t: int):
        """bf16 bits (q, k, v), each [S, D], of (batch b, query head h) at step t."""
        for tt, qkv in self.head_steps(b, h, t + 1):
            if tt == t:
                return qkv

    # ---- whole tensors --------------------------------------------------------
    def steps(self, n_steps: Optional[int] = None) -> Iterator[Tuple[int, np.ndarray, np.ndarray, np.ndarray]]:
        """Iterate (t, q, k, v) with bf16 bits shaped [batch, heads, S, D] (q)
        and [batch, kv_heads, S, D] (k, v)."""
        cfg = self.cfg
        T = cfg.steps if n_steps is None else n_steps
        G = cfg.group
        groups = [(b, g) for b in range(cfg.batch) for g in range(cfg.n_kv)]
        qshape = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
        kvshape = (cfg.batch, cfg.n_kv, cfg.seq_len, cfg.head_dim)
        with ThreadPoolExecutor(self.threads) as pool:
            def base(u):
                b, g = u
                q0s = [self.q_base(b, g * G + i) for i in range(G)]
                return q0s + self.kv_base(b, g, q0s)      # G queries, then k, v
            masters = list(pool.map(base, groups))

            def drift(iu, t):
                i, (b, g) = iu
                m = masters[i]
                for j in range(G):
                    m[j] = self._drift_one(m[j], _TENSOR_Q, b, g * G + j, t)
                m[G] = self._drift_one(m[G], _TENSOR_K, b, g, t)
                m[G + 1] = self._drift_one(m[G + 1], _TENSOR_V, b, g, t)

            for t in range(T):
                if t > 0:
                    list(pool.map(lambda iu: drift(iu, t), enumerate(groups)))
                qo = np.empty(qshape, dtype=np.uint16)
                ko = np.empty(kvshape, dtype=np.uint16)
                vo = np.empty(kvshape, dtype=np.uint16)

                def _round(iu):
                    i, (b, g) = iu
                    m = masters[i]
                    for j in range(G):
                        qo[b, g * G + j] = round_to_bf16_bits(m[j])
                    ko[b, g] = round_to_bf16_bits(m[G])
                    vo[b, g] = round_to_bf16_bits(m[G + 1])
                list(pool.map(_round, enumerate(groups)))
                yield t, qo, ko, vo
