"""Seeded synthetic inputs for the decode-step and SnapKV workloads.

This module draws inputs only: it holds none of the method's arithmetic and is the one
piece that both the GPU tests and the CPU oracle tests consume.  NumPy only.

Recipe (shapes from the pages' experiment setups: LLaMA-3-8B / Mistral-7B / LLaMA-3-70B
attention layers, 32K-128K contexts, 5-30 % budgets; SnapKV window 32, capacity 4096,
pool kernel 3):
  * generator ``numpy.random.Generator(PCG64(seed))``, seed = 1000 * config + step;
  * the projection P: a 128x32 standard-normal draw (fp64), reduced QR, columns signed so
    diag(R) > 0, rounded to fp32 -- a seeded random orthonormal stand-in for the learned
    projection;
  * q, K, V: standard-normal fp32 draws, rounded to bf16 (nearest-even);
  * outlier channels (32K / 128K configs): two distinct channels per KV head of the base
    key rows scaled by 8;
  * planted positions: drawn without replacement per KV head from the non-forced range
    [sink, n - local); their key rows become 3 * qhat_g + N(0, 0.3^2) where qhat_g is the
    unit mean of the group's query vectors (the window queries too for SnapKV).
bf16 arrays are returned as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D = 128
DP = 32
SINK = 4
LOCAL = 256

BUDGETS = {5: (1, 20), 10: (1, 10), 15: (3, 20), 20: (1, 5), 30: (3, 10), 100: (1, 1)}


def rng_for(config: int, step: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config + step))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 to bf16 (nearest, ties to even) and return uint16 bit patterns.
    In uint32: the largest finite pattern plus 0x8000 stays below 2^32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def projection(rng: np.random.Generator) -> np.ndarray:
    a = rng.standard_normal((D, DP))
    qm, r = np.linalg.qr(a)
    qm = qm * np.sign(np.diag(r))[None, :]
    return qm.astype(np.float32)


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _unit(v: np.ndarray) -> np.ndarray:
    return v / np.linalg.norm(v)


def plant_rows(rng, K_seq, qhat, count, sink=SINK, local=LOCAL):
    """Overwrite `count` key rows per KV head with 3*qhat_g + N(0, 0.3^2).  K_seq is the
    uint16 [n][Hkv][128] slice of one sequence (modified in place).  Returns positions."""
    n, Hkv, _ = K_seq.shape
    lo, hi = sink, n - local
    pos = []
    for g in range(Hkv):
        if hi <= lo or count <= 0:
            pos.append(np.zeros(0, np.int64))
            continue
        p = np.sort(rng.choice(hi - lo, size=min(count, hi - lo), replace=False) + lo)
        rows = 3.0 * qhat[g][None, :] + 0.3 * rng.standard_normal((len(p), D))
        K_seq[p, g, :] = f32_to_bf16_bits(rows.astype(np.float32))
        pos.append(p)
    return pos


@dataclass
class DecodeInputs:
    """One decode step's inputs.  K/V hold `capacity` rows per sequence in the packed
    layout given by `offsets` (n_b rows valid); P is the index projection."""
    config: int
    Hq: int
    Hkv: int
    offsets: np.ndarray          # int64 [B+1]
    q: np.ndarray                # uint16 [B][Hq][128]
    K: np.ndarray                # uint16 [Ntot][Hkv][128]
    V: np.ndarray                # uint16 [Ntot][Hkv][128]
    P: np.ndarray                # float32 [128][32]
    budget: tuple = (1, 5)
    planted: list = field(default_factory=list)

    @property
    def B(self) -> int:
        return len(self.offsets) - 1

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)


def group_qhat(q_b: np.ndarray, Hkv: int) -> np.ndarray:
    """Unit mean query direction per KV group, from bf16 bits q_b [Hq][128] (or
    [rows][Hq][128] for the SnapKV window)."""
    qf = bf16_bits_to_f32(q_b).astype(np.float64)
    if qf.ndim == 2:
        qf = qf[None]
    Hq = qf.shape[1]
    G = Hq // Hkv
    return np.stack([_unit(qf[:, g * G:(g + 1) * G, :].reshape(-1, D).mean(axis=0)) for g in range(Hkv)])


def make_decode(config: int, lengths, Hq: int, Hkv: int, planted_per_head, outliers: bool,
                budget=(1, 5), step: int = 0) -> DecodeInputs:
    rng = rng_for(config, step)
    P = projection(rng)
    lengths = [int(x) for x in lengths]
    B = len(lengths)
    offsets = np.zeros(B + 1, np.int64)
    offsets[1:] = np.cumsum(lengths)
    q = normal_bf16(rng, (B, Hq, D))
    Ntot = int(offsets[-1])
    K = np.empty((Ntot, Hkv, D), np.uint16)
    V = np.empty((Ntot, Hkv, D), np.uint16)
    planted = []
    for b in range(B):
        s, e = int(offsets[b]), int(offsets[b + 1])
        kf = rng.standard_normal((e - s, Hkv, D), dtype=np.float32)
        if outliers:
            for g in range(Hkv):
                ch = rng.choice(D, size=2, replace=False)
                kf[:, g, ch] *= 8.0
        K[s:e] = f32_to_bf16_bits(kf)
        del kf
        V[s:e] = normal_bf16(rng, (e - s, Hkv, D))
        cnt = planted_per_head(e - s) if callable(planted_per_head) else int(planted_per_head)
        planted.append(plant_rows(rng, K[s:e], group_qhat(q[b], Hkv), cnt))
    return DecodeInputs(config, Hq, Hkv, offsets, q, K, V, P, budget, planted)


def config1(step: int = 0) -> DecodeInputs:
    """Tiny decode step: 8 query / 2 KV heads, n = 4096, budget 10 %."""
    return make_decode(1, [4096], 8, 2, 32, False, BUDGETS[10], step)


def config2(step: int = 0, budget_pct: int = 20) -> DecodeInputs:
    """LLaMA-3-8B-shaped layer at n = 32768, two outlier channels per KV head."""
    return make_decode(2, [32768], 32, 8, 256, True, BUDGETS[budget_pct], step)


def config3(budget_pct: int = 20, n: int = 131072) -> DecodeInputs:
    """LLaMA-3-8B-shaped layer at n = 131072 (prefill state before the decode steps)."""
    return make_decode(3, [n], 32, 8, 256, True, BUDGETS[budget_pct], 0)


def config3_step(step: int, q_base: np.ndarray, Hkv: int = 8):
    """Decode step `step` >= 1: a fresh key/value row from the base distribution and a
    query q_base + N(0, 0.3^2).  Returns (q, k_new, v_new) as bf16 bits."""
    rng = rng_for(3, step)
    k_new = normal_bf16(rng, (1, Hkv, D))
    v_new = normal_bf16(rng, (1, Hkv, D))
    qf = bf16_bits_to_f32(q_base) + np.float32(0.3) * rng.standard_normal(q_base.shape, dtype=np.float32)
    return f32_to_bf16_bits(qf), k_new, v_new


def config4_lengths(B: int = 16) -> list:
    rng = rng_for(4, 0)
    return [int(x) for x in rng.integers(16384, 65536, size=B, endpoint=True)]


def config4(lengths=None) -> DecodeInputs:
    """Ragged batch of 16 sequences (Mistral-7B shapes), budget 15 %, 1 % planted."""
    if lengths is None:
        lengths = config4_lengths()
    return make_decode(4, lengths, 32, 8, lambda n: n // 100, False, BUDGETS[15], 1)


@dataclass
class SnapInputs:
    Hq: int
    Hkv: int
    q_obs: np.ndarray   # uint16 [w][Hq][128]
    K: np.ndarray       # uint16 [n][Hkv][128]
    V: np.ndarray
    c: int = 4096
    kernel: int = 3
    planted: list = field(default_factory=list)


def make_snap(config: int, n: int, w: int, Hq: int, Hkv: int, planted: int, c: int = 4096,
              kernel: int = 3, step: int = 0) -> SnapInputs:
    rng = rng_for(config, step)
    q_obs = normal_bf16(rng, (w, Hq, D))
    K = normal_bf16(rng, (n, Hkv, D))
    V = normal_bf16(rng, (n, Hkv, D))
    pos = plant_rows(rng, K, group_qhat(q_obs, Hkv), planted, sink=0, local=w)
    return SnapInputs(Hq, Hkv, q_obs, K, V, c, kernel, pos)


def config5(n: int = 131072) -> SnapInputs:
    """SnapKV at LLaMA-3-70B layer shapes: 64 query / 8 KV heads, w = 32, c = 4096."""
    return make_snap(5, n, 32, 64, 8, 512)
