"""Seeded synthetic Q, K, V.

Every draw comes from numpy's PCG64 seeded by a SeedSequence of small
integers, so the same (workload, seed) gives the same bits on any machine.
Values are drawn in fp32 and rounded once to the workload's dtype (bf16 with
round-to-nearest-even via torch's CPU conversion); those rounded bits are what
both the HIP path and the CPU oracle receive.

Recipe (video-DiT-shaped workloads):
  Q = Z_q + a_h * E,   K = Z_k + a_h * E,   V = Z_v,   Z ~ iid N(0, 1)
where E is a 3-D (t, y, x) sinusoidal position embedding projected to the head
dimension, and a_h is a per-head gain so that how concentrated a head's
attention is varies from head to head.  Unstructured workloads use iid N(0, 1)
for all three tensors.

Seeds: Z for (tensor, b, h) from SeedSequence([seed, wid, tensor, b, h]) with
tensor 0/1/2 = Q/K/V; gains a_h from SeedSequence([seed, wid, 99]); the
embedding projection from SeedSequence([seed, wid, 7]).
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os

import numpy as np
import torch

from .configs import Workload

_EMBED_FREQS = 16        # frequencies per axis
_EMBED_BASE = 100.0      # omega_f = base ** (-f / freqs)


def _rng(*words) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(x) for x in words])))


def head_gains(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-head gain a_h (float64, length H)."""
    rng = _rng(seed, w.wid, 99)
    lo, hi = w.gain_range
    if w.gain == "uniform":
        return rng.uniform(lo, hi, size=w.heads)
    if w.gain == "loguniform":
        return np.exp(rng.uniform(math.log(lo), math.log(hi), size=w.heads))
    raise ValueError(f"unknown gain law {w.gain!r}")


def make_embedding(w: Workload, seed: int = 0) -> np.ndarray:
    """E: [N, d] float32, rows rescaled to RMS w.embed_rms.

    Token n sits at (t, y, x) with n = (t*Y + y)*X + x (frame-major).  For each
    axis coordinate u and frequency f the features are sin(u*omega_f) and
    cos(u*omega_f); the 96 features are mapped to d dimensions by a fixed
    Gaussian matrix with variance 1/96.
    """
    T, Y, X = w.grid
    if T * Y * X < w.seq_len:
        raise ValueError(f"grid {w.grid} holds fewer than N={w.seq_len} tokens")
    n = np.arange(w.seq_len, dtype=np.int64)
    coords = (n // (Y * X), (n // X) % Y, n % X)
    omega = _EMBED_BASE ** (-np.arange(_EMBED_FREQS, dtype=np.float64) / _EMBED_FREQS)
    feats = []
    for u in coords:
        ang = u.astype(np.float64)[:, None] * omega[None, :]
        feats.append(np.sin(ang))
        feats.append(np.cos(ang))
    phi = np.concatenate(feats, axis=1)                       # [N, 96]
    nfeat = phi.shape[1]
    proj = _rng(seed, w.wid, 7).standard_normal((nfeat, w.head_dim)) / math.sqrt(nfeat)
    e = phi @ proj
    rms = np.sqrt(np.mean(e * e, axis=1, keepdims=True))
    e = e * (w.embed_rms / rms)
    return e.astype(np.float32)


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_inputs(w: Workload, seed: int = 0, threads: int | None = None):
    """Return (q, k, v) as contiguous CPU torch tensors [B, H, N, d] in w.dtype."""
    B, H, N, d = w.shape()
    dt = _torch_dtype(w.dtype)
    out = [torch.empty((B, H, N, d), dtype=dt) for _ in range(3)]
    emb = make_embedding(w, seed) if w.structured else None
    gains = head_gains(w, seed) if w.structured else None

    def fill(task):
        t, b, h = task
        z = _rng(seed, w.wid, t, b, h).standard_normal((N, d), dtype=np.float32)
        if emb is not None and t < 2:
            z += np.float32(gains[h]) * emb
        out[t][b, h].copy_(torch.from_numpy(z).to(dt))

    tasks = [(t, b, h) for t in range(3) for b in range(B) for h in range(H)]
    nthreads = threads or max(1, min(16, os.cpu_count() or 1))
    if nthreads == 1 or len(tasks) == 1:
        for task in tasks:
            fill(task)
    else:
        with cf.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, tasks))
    return tuple(out)
