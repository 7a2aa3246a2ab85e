"""Seeded synthetic workloads shaped like the OSCAR pages' decode workloads.

Every array is addressed by (workload, kind, request, head, chunk) so any
piece can be regenerated alone: a 100k-token batch never has to sit in host
memory whole, and a checker can rebuild only the requests it samples.

Value recipe (per KV head):
  * K and V rows ~ N(0, 1) in fp32 with a few fixed "outlier" channels
    multiplied by a large factor; which channels, how many and how large is
    drawn once per (workload, layer, KV head).
  * Each query head has covariance  Sigma = O diag(lam) O^T  with lam a
    geometric spectrum from 1 down to 1e-3 over head_dim entries and O a
    seeded Haar-random orthogonal matrix (QR of a Gaussian, sign fixed so the
    diagonal of the triangular factor is positive).
  * Calibration draws its own Q/K/V sequence from the same laws.
  * Tensors handed to the cache path are bf16 (fp32 rounded to nearest even)
    and are returned as uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096          # tokens per generator chunk
_TAG = 0x05CA2        # namespace for every SeedSequence of this module

KIND_K, KIND_V, KIND_Q, KIND_PROFILE, KIND_CALIB = 1, 2, 3, 4, 5
SHARED_REQUEST = 1 << 20   # request id used for positions inside a shared prefix


@dataclass(frozen=True)
class Workload:
    """One decode-layer workload (sizes only; no method parameters beyond
    the cache layout knobs the pages name)."""
    name: str
    index: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    batch: int
    context: int
    group: int = 32
    sink: int = 4
    recent: int = 128
    page_size: int = 16
    calib_tokens: int = 2048
    outliers: tuple = (4, 4)          # (min, max) outlier channels per head
    outlier_scale: tuple = (20.0, 20.0)  # (min, max) multiplier
    shared_prefix: int = 0            # tokens shared by every request (block-table sharing)
    write_chunk: int = 0              # tokens per timed quant_write chunk (0 = none)
    write_chunks: int = 0             # number of chunks per step for interleaved writes
    groups: tuple = field(default_factory=tuple)  # extra group sizes also run

    @property
    def gqa(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 1, 128, 1, 4096),
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 1, 32, 8, 128, 1, 32768, write_chunk=8192, write_chunks=1),
    "long_28x100k": Workload("long_28x100k", 2, 32, 8, 128, 28, 100_000,
                             outliers=(2, 6), outlier_scale=(10.0, 30.0)),
    "qwen3_32b_prefix": Workload("qwen3_32b_prefix", 3, 64, 8, 128, 64, 32768, shared_prefix=8192),
    "stress_16x128k": Workload("stress_16x128k", 4, 96, 8, 128, 16, 131072,
                               outlier_scale=(40.0, 40.0), write_chunk=4096, write_chunks=16,
                               groups=(32, 64)),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_TAG, *[int(k) & 0xFFFFFFFF for k in key]])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite by construction."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class HeadProfile:
    k_channels: np.ndarray   # outlier channel ids for K
    k_scales: np.ndarray
    v_channels: np.ndarray
    v_scales: np.ndarray


def head_profile(w: Workload, kv_head: int, layer: int = 0) -> HeadProfile:
    """Outlier channels and factors of one KV head (fixed for every request)."""
    g = _rng(w.index, KIND_PROFILE, layer, kv_head)
    out = []
    for _ in range(2):
        n = int(g.integers(w.outliers[0], w.outliers[1] + 1))
        ch = np.sort(g.choice(w.head_dim, size=n, replace=False)).astype(np.int64)
        sc = g.uniform(w.outlier_scale[0], w.outlier_scale[1], size=n) if w.outlier_scale[0] != w.outlier_scale[1] \
            else np.full(n, w.outlier_scale[0])
        out += [ch, sc.astype(np.float32)]
    return HeadProfile(*out)


_Q_FACTORS: dict = {}


def q_factor(w: Workload, q_head: int, layer: int = 0) -> np.ndarray:
    """Matrix F with rows q = z F, z ~ N(0, I), so Cov(q) = F^T F = O diag(lam) O^T.
    Deterministic in (workload, head, layer); kept after the first call (read-only)."""
    key = (w, q_head, layer)
    f = _Q_FACTORS.get(key)
    if f is None:
        f = _q_factor(w, q_head, layer)
        f.setflags(write=False)
        _Q_FACTORS[key] = f
    return f


def _q_factor(w: Workload, q_head: int, layer: int) -> np.ndarray:
    d = w.head_dim
    g = _rng(w.index, KIND_Q, layer, q_head, 0xFFFF)
    a = g.standard_normal((d, d))
    o, r = np.linalg.qr(a)
    o = o * np.sign(np.diag(r))[None, :]
    lam = np.geomspace(1.0, 1e-3, d)
    return (np.sqrt(lam)[:, None] * o.T)           # F = diag(sqrt lam) O^T


def _kv_rows(g: np.random.Generator, n: int, d: int, ch: np.ndarray, sc: np.ndarray) -> np.ndarray:
    x = g.standard_normal((n, d), dtype=np.float32)
    x[:, ch] *= sc[None, :]
    return x


def kv_chunk_f32(w: Workload, kind: int, request: int, kv_head: int, chunk: int, layer: int = 0) -> np.ndarray:
    """fp32 rows [CHUNK, head_dim] for positions chunk*CHUNK ... of one request/head.
    Positions inside a shared prefix come from the shared request id."""
    if w.shared_prefix and (chunk + 1) * CHUNK <= w.shared_prefix:
        request = SHARED_REQUEST
    prof = head_profile(w, kv_head, layer)
    ch, sc = (prof.k_channels, prof.k_scales) if kind == KIND_K else (prof.v_channels, prof.v_scales)
    g = _rng(w.index, kind, layer, request, kv_head, chunk)
    return _kv_rows(g, CHUNK, w.head_dim, ch, sc)


def kv_tokens_bf16(w: Workload, kind: int, request: int, kv_head: int, start: int, stop: int,
                   layer: int = 0) -> np.ndarray:
    """bf16 bits [stop-start, head_dim] for positions [start, stop) of one request/head."""
    out = np.empty((stop - start, w.head_dim), dtype=np.uint16)
    c0, c1 = start // CHUNK, (stop - 1) // CHUNK if stop > start else start // CHUNK - 1
    for c in range(c0, c1 + 1):
        rows = f32_to_bf16_bits(kv_chunk_f32(w, kind, request, kv_head, c, layer))
        a, b = max(start, c * CHUNK), min(stop, (c + 1) * CHUNK)
        out[a - start:b - start] = rows[a - c * CHUNK:b - c * CHUNK]
    return out


def kv_request_bf16(w: Workload, request: int, start: int, stop: int, layer: int = 0,
                    threads: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """K and V bf16 bits [stop-start, n_kv_heads, head_dim] for one request."""
    n = stop - start
    k = np.empty((n, w.n_kv_heads, w.head_dim), dtype=np.uint16)
    v = np.empty_like(k)

    def job(args):
        kind, h = args
        dst = k if kind == KIND_K else v
        dst[:, h, :] = kv_tokens_bf16(w, kind, request, h, start, stop, layer)

    jobs = [(kind, h) for kind in (KIND_K, KIND_V) for h in range(w.n_kv_heads)]
    nthreads = threads or min(16, len(os.sched_getaffinity(0)))
    if nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(job, jobs))
    else:
        for j in jobs:
            job(j)
    return k, v


def q_decode_bf16(w: Workload, request: int, step: int = 0, layer: int = 0) -> np.ndarray:
    """bf16 bits [n_q_heads, head_dim]: the decode query of one request."""
    q = np.empty((w.n_q_heads, w.head_dim), dtype=np.float32)
    for h in range(w.n_q_heads):
        g = _rng(w.index, KIND_Q, layer, request, h, step)
        q[h] = (g.standard_normal(w.head_dim) @ q_factor(w, h, layer)).astype(np.float32)
    return f32_to_bf16_bits(q)


def q_batch_bf16(w: Workload, step: int = 0, layer: int = 0) -> np.ndarray:
    return np.stack([q_decode_bf16(w, r, step, layer) for r in range(w.batch)])


def calib_samples(w: Workload, kv_head: int, layer: int = 0, n: int | None = None):
    """Calibration sequence of one KV head: fp32 Q [n, gqa, d], K [n, d], V [n, d]."""
    n = n or w.calib_tokens
    prof = head_profile(w, kv_head, layer)
    g = _rng(w.index, KIND_CALIB, layer, kv_head)
    k = _kv_rows(g, n, w.head_dim, prof.k_channels, prof.k_scales)
    v = _kv_rows(g, n, w.head_dim, prof.v_channels, prof.v_scales)
    q = np.empty((n, w.gqa, w.head_dim), dtype=np.float32)
    for j in range(w.gqa):
        hq = kv_head * w.gqa + j
        q[:, j, :] = (g.standard_normal((n, w.head_dim)) @ q_factor(w, hq, layer)).astype(np.float32)
    return q, k, v


def calib_layer(w: Workload, layer: int = 0, n: int | None = None):
    """Calibration arrays of every KV head: Q [n, Hq, d], K [n, Hkv, d], V [n, Hkv, d] (fp32)."""
    qs, ks, vs = zip(*[calib_samples(w, h, layer, n) for h in range(w.n_kv_heads)])
    q = np.concatenate(qs, axis=1)  # heads ordered kv_head-major, matching q head ids
    return np.ascontiguousarray(q), np.ascontiguousarray(np.stack(ks, 1)), np.ascontiguousarray(np.stack(vs, 1))
