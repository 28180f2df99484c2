"""Seeded generator of post-RoPE Q, K, V for one attention layer.

Structure (the ProxyAttn blog post, ir.hit.edu.cn, section 3 "观察"): all
heads look at the same places (a shared latent sequence z) but differ in how
sharply they focus (a per-head scale beta_h); a few planted "needle" keys
along a direction v are matched by a fraction of the queries.

For each workload (see ``configs.py``):

* z_t ~ N(0, I_d) for t in [0, N); with ``group_latent_corr`` = c each KV head
  kappa instead has z^(kappa) = sqrt(c) * s + sqrt(1-c) * u^(kappa) with s, u
  independent N(0, I_d) sequences (correlation c between KV groups).
* K[kappa, t] = z^(kappa)_t + 0.5 * eps'_{kappa,t} (+ 4 v at needle positions).
* Q[h, t] = beta_h * (z^(kv(h))_{t-1} + 0.5 * eps_{h,t} (+ 3 v at needle
  queries)), with z_{-1} read as z_0 (lag-1 match), beta_h log-uniform.
* V[kappa, t] ~ N(0, I_d).
* Rotary embedding (rotate-half form, inv_freq_i = base^(-2i/d), angles in
  float64) on Q and K when the workload names a base.
* Storage: IEEE float32 for the fp32 workload; otherwise round-to-nearest-even
  bfloat16 (returned as uint16 bit patterns).

kv(h) = h // (H / Hkv) (consecutive query heads share a KV head).

Every random draw comes from a child stream of ``numpy.random.SeedSequence``
(seed), so heads can be filled in parallel threads and the result does not
depend on the thread count.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

from .configs import WorkloadConfig


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact float32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads(threads: Optional[int]) -> int:
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class _Streams:
    """Named child streams of one SeedSequence (fixed spawn layout)."""

    def __init__(self, cfg: WorkloadConfig):
        root = np.random.SeedSequence(cfg.seed)
        params, latent, knoise, qnoise, vals = root.spawn(5)
        self.params = np.random.default_rng(params)
        self.latent = [np.random.default_rng(s) for s in latent.spawn(1 + cfg.num_kv_heads)]
        self.knoise = [np.random.default_rng(s) for s in knoise.spawn(cfg.num_kv_heads)]
        self.qnoise = [np.random.default_rng(s) for s in qnoise.spawn(cfg.num_heads)]
        self.vals = [np.random.default_rng(s) for s in vals.spawn(cfg.num_kv_heads)]


def draw_params(cfg: WorkloadConfig, streams: Optional[_Streams] = None) -> Dict[str, np.ndarray]:
    """Per-head beta, needle direction v and the needle key / query positions."""
    g = (streams or _Streams(cfg)).params
    lo, hi = cfg.beta_range
    beta = np.exp(g.uniform(np.log(lo), np.log(hi), size=cfg.num_heads))
    v = g.standard_normal(cfg.head_dim)
    v /= np.linalg.norm(v)
    n_q = int(round(cfg.needle_query_frac * cfg.seq_len))
    needle_keys = np.sort(g.choice(cfg.seq_len, size=cfg.n_needles, replace=False))
    needle_queries = np.sort(g.choice(cfg.seq_len, size=n_q, replace=False))
    return {"beta": beta, "v": v, "needle_keys": needle_keys, "needle_queries": needle_queries}


def _rope_tables(cfg: WorkloadConfig):
    d = cfg.head_dim
    inv_freq = cfg.rope_base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.arange(cfg.seq_len, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def _apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half rotary embedding of x [N, d] (float64 arithmetic)."""
    h = x.shape[1] // 2
    x = x.astype(np.float64)
    out = np.empty_like(x)
    out[:, :h] = x[:, :h] * cos - x[:, h:] * sin
    out[:, h:] = x[:, h:] * cos + x[:, :h] * sin
    return out


def generate(cfg: WorkloadConfig, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Return {"q": [H,N,d], "k": [Hkv,N,d], "v": [Hkv,N,d], "params": ...}.

    Arrays are float32 when ``cfg.dtype == "fp32"``, else uint16 bfloat16 bits.
    """
    H, Hkv, d, N = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.seq_len
    if H % Hkv:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    st = _Streams(cfg)
    p = draw_params(cfg, st)
    v = p["v"].astype(np.float32)
    rope = _rope_tables(cfg) if cfg.rope_base else None
    bf16 = cfg.dtype != "fp32"
    out_dtype = np.uint16 if bf16 else np.float32

    # Latent sequences, one per KV head (shared unless group_latent_corr is set).
    if cfg.group_latent_corr is None:
        z0 = st.latent[0].standard_normal((N, d), dtype=np.float32)
        latents = [z0] * Hkv
    else:
        c = cfg.group_latent_corr
        s = st.latent[0].standard_normal((N, d), dtype=np.float32)
        latents = []
        for kv in range(Hkv):
            u = st.latent[1 + kv].standard_normal((N, d), dtype=np.float32)
            latents.append((np.float32(np.sqrt(c)) * s + np.float32(np.sqrt(1.0 - c)) * u).astype(np.float32))

    q = np.empty((H, N, d), dtype=out_dtype)
    k = np.empty((Hkv, N, d), dtype=out_dtype)
    vv = np.empty((Hkv, N, d), dtype=out_dtype)
    qpos = p["needle_queries"]
    kpos = p["needle_keys"]
    grp = H // Hkv

    def store(dst, x):
        if rope is not None:
            x = _apply_rope(x, *rope).astype(np.float32)
        dst[...] = f32_to_bf16_bits(x) if bf16 else x.astype(np.float32)

    def make_k(kv):
        x = latents[kv] + np.float32(0.5) * st.knoise[kv].standard_normal((N, d), dtype=np.float32)
        x[kpos] += np.float32(4.0) * v
        store(k[kv], x)

    def make_q(h):
        z = latents[h // grp]
        x = np.empty((N, d), dtype=np.float32)
        x[1:] = z[:-1]
        x[0] = z[0]
        x += np.float32(0.5) * st.qnoise[h].standard_normal((N, d), dtype=np.float32)
        x[qpos] += np.float32(3.0) * v
        x *= np.float32(p["beta"][h])
        store(q[h], x)

    def make_v(kv):
        x = st.vals[kv].standard_normal((N, d), dtype=np.float32)
        vv[kv] = f32_to_bf16_bits(x) if bf16 else x

    jobs = [(make_k, i) for i in range(Hkv)] + [(make_q, i) for i in range(H)] + \
           [(make_v, i) for i in range(Hkv)]
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(lambda j: j[0](j[1]), jobs))
    return {"q": q, "k": k, "v": vv, "params": p}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round an fp32 workload's tensors once to bfloat16 (bf16 ones pass through)."""
    return x if x.dtype == np.uint16 else f32_to_bf16_bits(x)


def input_digest(*arrays: np.ndarray) -> str:
    """SHA-256 over the raw bytes of the given arrays (for logging)."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
