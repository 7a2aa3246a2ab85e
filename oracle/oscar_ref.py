"""Plain fp64 CPU oracle for the OSCAR 2-bit KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke entry point and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product.

It is written from the three pages on OSCAR ("Offline Spectral
Covariance-Aware Rotation", arXiv 2605.17757).  Citation keys:

  [IT]  gist.science, Italian technical summary "Riepilogo Tecnico: OSCAR -
        Rotazione Consapevole della Covarianza Spettrale Offline ..."
        (sections 1-5; calibration in 2.2.A, serving in 2.2.B).
  [ES]  7minutos.es news article "... OSCAR: un sistema de cuantificacion de
        cache KV de 2 bits consciente de la atencion ..." (sections "Lo que
        OSCAR hace diferente" and "El sistema de servicio: diseno de cache de
        precision mixta").
  [JA]  gist.science, Japanese technical summary (same structure as [IT]).

Everything is numpy float64 unless a page or the storage format fixes a
narrower type (bf16 inputs, fp32 rotations and thresholds, fp16 scale/zero,
2-bit codes).  Readings of points the pages leave open are marked READING.

Pinned by tests/test_oracle_pins.py (identities, closed forms, brute force,
special cases reducing to library routines, the pages' printed constants) and
tests/test_oracle_pins_calibration.py (the composite rotation's closed form,
the clip threshold's quantile and pooling, the query heads of a KV head).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

PAGE = 16          # tokens per cache page (storage format)


# ---------------------------------------------------------------------------
# dtype helpers (input decoding; the oracle's own, independent of the product)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 to IEEE binary16, nearest-even, in a single rounding
    (numpy converts from the double's bits directly; pinned in the tests
    against exact rational arithmetic)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# 8-bit scale and zero of the lower-metadata history format: the OCP FP8 E4M3
# encoding (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
# subnormal; S.1111.111 is NaN; no infinities; largest finite 448).
E4M3_NAN = np.uint8(0x7F)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """FP8 E4M3 codes (uint8) -> exact float64 values."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


_E4M3_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))   # codes 0x00..0x7E: 0 .. 448, increasing


def to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float64 to FP8 E4M3, nearest with ties to the even code, in a
    single rounding; the sign is kept (so -0.0 -> 0x80).  READING: magnitudes
    beyond 448 saturate to 448 (the format has no infinity); NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(_E4M3_POS, a), 1, 0x7E)       # _E4M3_POS[i-1] < a <= _E4M3_POS[i]
    lo, hi = _E4M3_POS[i - 1], _E4M3_POS[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    code = np.where(pick_hi, i, i - 1)
    code = np.where(a >= 448.0, 0x7E, code)
    code = np.where(a == 0, 0, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return np.where(np.isnan(x), E4M3_NAN, code).astype(np.uint8)


# ---------------------------------------------------------------------------
# The fixed parts of the composite rotation  ([ES] "Lo que OSCAR hace
# diferente": Lemma 1 and the bit-reversal paragraph; [IT] 2.2.A)
# ---------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    """Orthonormal Walsh-Hadamard matrix of size d (a power of two), Sylvester
    construction in natural order: H[i, j] = (-1)^popcount(i & j) / sqrt(d).
    READING: natural (not sequency) order and full size d; Lemma 1's tr/d
    value needs the full orthonormal matrix."""
    assert d > 0 and d & (d - 1) == 0
    i = np.arange(d)
    parity = np.zeros((d, d), dtype=np.int64)
    a = i[:, None] & i[None, :]
    while np.any(a):
        parity ^= a & 1
        a = a >> 1
    return np.where(parity == 1, -1.0, 1.0) / math.sqrt(d)


def bit_reverse(j: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (j & 1)
        j >>= 1
    return r


def bitrev_perm(d: int) -> np.ndarray:
    """Permutation matrix P_br with P[i, j] = 1 iff i is the bit reversal of j.
    With row vectors, (x P)[j] = x[rev(j)]: output channel j reads input
    channel rev(j), so each power-of-two group of outputs draws one channel
    from every importance stratum of the input ([ES], bit-reversal paragraph)."""
    bits = d.bit_length() - 1
    p = np.zeros((d, d))
    for j in range(d):
        p[bit_reverse(j, bits), j] = 1.0
    return p


# ---------------------------------------------------------------------------
# Offline calibration ([IT] 2.2.A; [ES] "Lo que OSCAR hace diferente"; [JA] 2.2.A)
# ---------------------------------------------------------------------------

def query_covariance(q: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n, uncentred, q_n row vectors.
    q: [N, g, d] -- the g query heads that read one KV head are pooled
    (READING: summing the logit-error identity over the heads that share a
    key gives the pooled weight), so N counts N*g rows."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, q.shape[-1])
    return q.T @ q / q.shape[0]


def causal_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """S = row-softmax(Q K^T / sqrt(d)) with row n seeing keys 0..n (causal)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    n, d = q.shape
    logits = q @ k.T / math.sqrt(d)
    logits[np.triu_indices(n, 1)] = -np.inf
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return e / e.sum(axis=1, keepdims=True)


def score_weighted_value_covariance(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V for each query head of the group, pooled over
    the g heads like C_Q.  q: [N, g, d]; k, v: [N, d] (unquantised)."""
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, g, _ = q.shape
    c = np.zeros((v.shape[1], v.shape[1]))
    for h in range(g):
        s = causal_scores(q[:, h, :], k)
        c += v.T @ s.T @ s @ v
    return c / (n * g)


def eig_desc(c: np.ndarray):
    """Eigen-decomposition of a symmetric matrix, eigenvalues descending.
    READING (sign convention, pages silent): each eigenvector is flipped so
    that its entry of largest magnitude is positive (ties: lowest index)."""
    lam, u = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(-lam, kind="stable")
    lam, u = lam[order], u[:, order].copy()
    for j in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, j])))
        if u[i, j] < 0:
            u[:, j] = -u[:, j]
    return lam, u


def composite_rotation(u: np.ndarray) -> np.ndarray:
    """R = U H_Had P_br ([IT] 2.2.A formula; [ES] composite rotations)."""
    d = u.shape[0]
    return u @ hadamard(d) @ bitrev_perm(d)


def quantile_linear(values: np.ndarray, c: float) -> float:
    """c-quantile with linear interpolation between order statistics."""
    return float(np.quantile(np.asarray(values, dtype=np.float64).ravel(), c, method="linear"))


@dataclass
class LayerCalibration:
    r_k: np.ndarray      # [Hkv, d, d] float32  (x_rot = x @ R)
    r_v: np.ndarray      # [Hkv, d, d] float32
    eig_k: np.ndarray    # [Hkv, d] eigenvalues of C_Q, descending
    eig_v: np.ndarray    # [Hkv, d] eigenvalues of C_S, descending
    tau_k: np.float32
    tau_v: np.float32


ROTATIONS = ("oscar", "identity", "hadamard")


def calibrate_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    clip_k: float = 0.96, clip_v: float = 0.92, rotation: str = "oscar") -> LayerCalibration:
    """Offline calibration of one layer.
    q: [N, Hq, d]; k, v: [N, Hkv, d] calibration activations (fp32 values).
    Per KV head: C_Q and C_S, their eigenbases, R_K = U_Q H P_br and
    R_V = U_S H P_br, stored as fp32.  Per layer: clip thresholds
    ([ES] write path: percentile threshold, typical c_K = 0.96, c_V = 0.92).
    READING: tau is the c-quantile of |x R| over all calibration tokens, KV
    heads and channels of the layer, computed with the stored fp32 R.
    rotation: "oscar" (the above), or one of the pages' baselines ([ES]
    accuracy paragraph and the paragraph before "Lo que OSCAR hace
    diferente"; [IT] 4): "identity", naive INT2 with no rotation (R = I), and
    "hadamard", the data-oblivious Hadamard rotation (R = H P_br, the
    composite with U = I).  Neither baseline looks at the covariances; their
    eig arrays are NaN.  tau is recomputed for the chosen R."""
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {ROTATIONS}")
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    r_k = np.empty((hkv, d, d), dtype=np.float32)
    r_v = np.empty_like(r_k)
    eig_k = np.full((hkv, d), np.nan)
    eig_v = np.full((hkv, d), np.nan)
    rot_k, rot_v = [], []
    for h in range(hkv):
        if rotation == "oscar":
            qh = q[:, h * g:(h + 1) * g, :]
            lam_q, u_q = eig_desc(query_covariance(qh))
            lam_s, u_s = eig_desc(score_weighted_value_covariance(qh, k[:, h, :], v[:, h, :]))
            r_k[h] = composite_rotation(u_q).astype(np.float32)
            r_v[h] = composite_rotation(u_s).astype(np.float32)
            eig_k[h], eig_v[h] = lam_q, lam_s
        elif rotation == "hadamard":
            r_k[h] = r_v[h] = composite_rotation(np.eye(d)).astype(np.float32)
        else:
            r_k[h] = r_v[h] = np.eye(d, dtype=np.float32)
        rot_k.append(np.abs(k[:, h, :].astype(np.float64) @ r_k[h].astype(np.float64)))
        rot_v.append(np.abs(v[:, h, :].astype(np.float64) @ r_v[h].astype(np.float64)))
    tau_k = np.float32(quantile_linear(np.concatenate(rot_k), clip_k))
    tau_v = np.float32(quantile_linear(np.concatenate(rot_v), clip_v))
    return LayerCalibration(r_k, r_v, eig_k, eig_v, tau_k, tau_v)


# ---------------------------------------------------------------------------
# Write path: rotate, clip, per-token asymmetric INT2 per channel group
# ([ES] write path paragraph; [IT] 2.2.B)
# ---------------------------------------------------------------------------

F16_NAN = np.float16(np.nan)


def quantize(x: np.ndarray, r: np.ndarray, tau: float, group: int, scale_bits: int = 16):
    """x: [n, d] input values (bf16 values as float64), r: [d, d] (fp32 values),
    tau: clip threshold (fp32 value).  Returns codes uint8 [n, d],
    scale/zero [n, d/group] and the rotated, clipped fp64 values.
    Steps (all fp64 until the rounding of scale and zero):
      x_rot = x R ; clamp to [-tau, tau] ;
      per group: mn, mx ; s = f16((mx - mn) / 3) ; z = f16(mn) ;
      c = clamp(round_half_even((x_rot - z) / s), 0, 3), c = 0 where s == 0.
    READING: codes are taken against the rounded s and z, so the encoder and
    the decoder (z + c s) agree.  A group holding NaN stores s = z = NaN and
    codes 0.  scale_bits = 16 stores s and z as float16; scale_bits = 8 (the
    lower-metadata format) as FP8 E4M3 codes (uint8), the same steps with
    e4m3 rounding in place of f16."""
    if scale_bits not in (16, 8):
        raise ValueError("scale_bits must be 16 or 8")
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    ng = d // group
    xr = x @ np.asarray(r, dtype=np.float64)
    t = float(tau)
    xr = np.clip(xr, -t, t)
    xg = xr.reshape(n, ng, group)
    mn = xg.min(axis=2)
    mx = xg.max(axis=2)
    if scale_bits == 16:
        s = to_f16((mx - mn) / 3.0)
        z = to_f16(mn)
    else:
        s = to_e4m3((mx - mn) / 3.0)
        z = to_e4m3(mn)
    s64 = meta_values(s)[:, :, None]
    z64 = meta_values(z)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        tt = (xg - z64) / s64
    c = np.clip(np.rint(tt), 0, 3)
    bad = np.isnan(mn) | np.isnan(mx)
    c = np.where((s64 == 0) | bad[:, :, None], 0, c)
    nan = F16_NAN if scale_bits == 16 else E4M3_NAN
    s = np.where(bad, nan, s)
    z = np.where(bad, nan, z)
    return c.reshape(n, d).astype(np.uint8), s, z, xr


def meta_values(m: np.ndarray) -> np.ndarray:
    """Stored scale or zero -> float64: float16 values, or E4M3 codes (uint8)."""
    m = np.asarray(m)
    return e4m3_decode(m) if m.dtype == np.uint8 else m.astype(np.float64)


def dequantize(codes: np.ndarray, s: np.ndarray, z: np.ndarray, group: int) -> np.ndarray:
    """Rotated-basis reconstruction z + c s (fp64)."""
    n, d = codes.shape
    c = codes.astype(np.float64).reshape(n, d // group, group)
    return (meta_values(z)[:, :, None] + c * meta_values(s)[:, :, None]).reshape(n, d)


def unrotate(x_rot: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Back to the original basis with R^T (R orthogonal)."""
    return np.asarray(x_rot, dtype=np.float64) @ np.asarray(r, dtype=np.float64).T


# ---------------------------------------------------------------------------
# Mixed-precision layout: regions of a request  ([ES] serving section:
# sink, recent and history regions; [IT] 2.2.B)
# ---------------------------------------------------------------------------

REGION_SINK, REGION_INT2, REGION_RECENT = 0, 1, 2


def regions(t: int, sink: int, recent: int) -> np.ndarray:
    """Region of every position 0..t-1 for a request of length t: the first
    `sink` positions and the last `recent` positions stay bf16, the rest is
    INT2.  READING: the recent window is the last `recent` positions
    including the newest token; if t <= sink + recent everything is bf16."""
    p = np.arange(t)
    reg = np.full(t, REGION_INT2, dtype=np.int8)
    reg[p < sink] = REGION_SINK
    reg[(p >= sink) & (p >= t - recent)] = REGION_RECENT
    return reg


def bits_per_element(t: int, sink: int, recent: int, history_bits: float, bf16_bits: float = 16.0) -> float:
    """Average stored bits per KV element over a request of length t."""
    n_bf16 = min(t, sink + recent)
    return (n_bf16 * bf16_bits + (t - n_bf16) * history_bits) / t


def int2_history_bits(group: int, scale_bits: int = 16, zero_bits: int = 16) -> float:
    return 2.0 + (scale_bits + zero_bits) / group


# ---------------------------------------------------------------------------
# Decode attention, exact fp64, basis-free ([IT] 2.2.B read path)
# ---------------------------------------------------------------------------

def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q: [Hq, d]; k, v: [T, Hkv, d] (the values the cache represents, in the
    original basis).  Query head h reads KV head h // (Hq/Hkv).
    o_h = sum_t softmax_t(q_h . k_t / sqrt(d)) v_t.  T = 0 gives zeros."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    t, hkv, _ = k.shape
    out = np.zeros((hq, d))
    if t == 0:
        return out
    g = hq // hkv
    for h in range(hq):
        kh = np.asarray(k[:, h // g, :], dtype=np.float64)
        vh = np.asarray(v[:, h // g, :], dtype=np.float64)
        logit = kh @ q[h] / math.sqrt(d)
        logit -= logit.max()
        p = np.exp(logit)
        out[h] = (p / p.sum()) @ vh
    return out


@dataclass
class StoredRequest:
    """What the cache holds for one request (per position and KV head)."""
    region: np.ndarray        # [T] int8
    k_bf16: np.ndarray        # [T, Hkv, d] uint16 (meaningful for bf16 positions)
    v_bf16: np.ndarray
    k_codes: np.ndarray       # [T, Hkv, d] uint8 (meaningful for INT2 positions)
    k_s: np.ndarray           # [T, Hkv, NG] float16
    k_z: np.ndarray
    v_codes: np.ndarray
    v_s: np.ndarray
    v_z: np.ndarray


def store_request(k_bits: np.ndarray, v_bits: np.ndarray, cal: LayerCalibration, group: int,
                  sink: int, recent: int, scale_bits: int = 16) -> StoredRequest:
    """Apply the region rule and the write path to a whole request.
    k_bits, v_bits: [T, Hkv, d] bf16 bit patterns."""
    t, hkv, d = k_bits.shape
    ng = d // group
    reg = regions(t, sink, recent)
    kc = np.zeros((t, hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.zeros((t, hkv, ng), np.float16 if scale_bits == 16 else np.uint8)
    kz, vs, vz = ks.copy(), ks.copy(), ks.copy()
    idx = np.nonzero(reg == REGION_INT2)[0]
    if idx.size:
        for h in range(hkv):
            c, s, z, _ = quantize(bf16_to_f64(k_bits[idx, h]), cal.r_k[h], cal.tau_k, group, scale_bits)
            kc[idx, h], ks[idx, h], kz[idx, h] = c, s, z
            c, s, z, _ = quantize(bf16_to_f64(v_bits[idx, h]), cal.r_v[h], cal.tau_v, group, scale_bits)
            vc[idx, h], vs[idx, h], vz[idx, h] = c, s, z
    return StoredRequest(reg, k_bits, v_bits, kc, ks, kz, vc, vs, vz)


def represented_kv(st: StoredRequest, cal: LayerCalibration, group: int):
    """Original-basis K, V the cache represents: bf16 values for bf16
    positions, (z + c s) R^T for INT2 positions (explicit inverse rotation)."""
    k = bf16_to_f64(st.k_bf16)
    v = bf16_to_f64(st.v_bf16)
    idx = np.nonzero(st.region == REGION_INT2)[0]
    for h in range(k.shape[1]):
        if idx.size:
            k[idx, h] = unrotate(dequantize(st.k_codes[idx, h], st.k_s[idx, h], st.k_z[idx, h], group), cal.r_k[h])
            v[idx, h] = unrotate(dequantize(st.v_codes[idx, h], st.v_s[idx, h], st.v_z[idx, h], group), cal.r_v[h])
    return k, v


def decode_attention(q_bits: np.ndarray, st: StoredRequest, cal: LayerCalibration, group: int) -> np.ndarray:
    """Exact fp64 decode attention of one request over its mixed cache.
    q_bits: [Hq, d] bf16 bit patterns."""
    k, v = represented_kv(st, cal, group)
    return attend(bf16_to_f64(q_bits), k, v)


def prefill_attention(q_bits: np.ndarray, st: StoredRequest, cal: LayerCalibration, group: int) -> np.ndarray:
    """Exact fp64 attention of a chunk of C new queries over the mixed cache
    (chunked prefill, [IT] 2.2.B / [ES] serving section: prefix-cached chunked
    prefill over the same paged cache).  st holds the request after the
    chunk's C tokens were written, T positions in all; query c sits at
    position T - C + c and attends the positions up to and including its own
    (causal), each in the form the cache holds it.  q_bits: [C, Hq, d] bf16
    bit patterns; returns [C, Hq, d]."""
    k, v = represented_kv(st, cal, group)
    c_n = q_bits.shape[0]
    t = k.shape[0]
    return np.stack([attend(bf16_to_f64(q_bits[c]), k[:t - c_n + c + 1], v[:t - c_n + c + 1])
                     for c in range(c_n)])


# ---------------------------------------------------------------------------
# Storage format of one page (per KV head).  Written out independently here
# from the format's definition so stored bytes can be compared exactly.
#
# INT2 page block, d channels, NG = d / G groups, 16 tokens:
#   [0, 16*d/4)          K codes, token-major: token t owns d/4 bytes, each
#                        byte four 2-bit fields (field m at bits 2*m); which
#                        channel each field holds is k_code_channel below.
#   next 16*NG*4 bytes   K scale/zero as fp16 pairs, token-major [16][NG][(s, z)].
#   next 16*d/4 bytes    V codes, [4][d] bytes by token quad: byte [q][j]
#                        holds channel j of tokens 4q..4q+3, token 4q+i at
#                        bits 2*i.
#   next 16*NG*4 bytes   V scale/zero as fp16 pairs, group-major [NG][16][(s, z)].
# BF16 page block: K as [16][d] bf16 (token-major), then V as [d][16] bf16
# (channel-major).
# ---------------------------------------------------------------------------

def k_code_channel(d: int, group: int) -> np.ndarray:
    """Channel held by each 2-bit field of a token's K-code bytes: entry
    4*b + m is the channel at bits 2*m of byte b.

    d = 128: byte b = 8*a + 4*w + i is byte i of word w of quarter a, and
    every field position of a word belongs to one group:
      G = 32: field m holds channel 64*w + 32*(m // 2) + 8*a + 4*(m % 2) + i
              (fields 0, 1: group 2*w; fields 2, 3: group 2*w + 1);
      G = 64: field m holds channel 64*w + 16*a + 4*m + i (word w: group w).
    Other shapes: channels run consecutively, channel j in byte j // 4 at
    field j % 4."""
    field = np.arange(d)
    b, m = field // 4, field % 4
    a, w, i = b // 8, (b // 4) % 2, b % 4
    if d == 128 and group == 32:
        return 64 * w + 32 * (m // 2) + 8 * a + 4 * (m % 2) + i
    if d == 128 and group == 64:
        return 64 * w + 16 * a + 4 * m + i
    return field


def int2_block_bytes(d: int, group: int, scale_bits: int = 16) -> int:
    return 2 * (PAGE * d // 4 + PAGE * (d // group) * scale_bits // 4)


def bf16_block_bytes(d: int) -> int:
    return 2 * PAGE * d * 2


def _pack_sz(s: np.ndarray, z: np.ndarray, token_major: bool) -> np.ndarray:
    # s, z: [16, NG] float16 or E4M3 codes -> bytes of [16][NG][(s, z)]
    # (token-major) or [NG][16][(s, z)]: a float16 pair, or a byte pair
    pair = np.stack([s, z] if token_major else [s.T, z.T], axis=-1)
    pair = pair.astype(np.uint8 if pair.dtype == np.uint8 else np.float16)
    return np.ascontiguousarray(pair).view(np.uint8).ravel()


def pack_int2_block(kc, ks, kz, vc, vs, vz) -> np.ndarray:
    """Codes [16, d] (uint8 0..3), scale/zero [16, NG] (float16, or uint8 E4M3
    codes for the lower-metadata format) -> uint8 block."""
    kc = np.asarray(kc, np.uint8)
    vc = np.asarray(vc, np.uint8)
    t, d = kc.shape
    assert t == PAGE
    ng = np.asarray(ks).shape[1]
    kf = kc[:, k_code_channel(d, d // ng)]          # field 4*b + m of each token
    kbytes = np.zeros((PAGE, d // 4), np.uint8)
    for m in range(4):
        kbytes |= (kf[:, m::4] << (2 * m)).astype(np.uint8)
    vbytes = np.zeros((4, d), np.uint8)
    for q in range(4):
        for i in range(4):
            vbytes[q] |= (vc[4 * q + i, :] << (2 * i)).astype(np.uint8)
    return np.concatenate([kbytes.ravel(), _pack_sz(ks, kz, True), vbytes.ravel(),
                           _pack_sz(vs, vz, False)])


def unpack_int2_block(buf: np.ndarray, d: int, group: int, scale_bits: int = 16):
    """Inverse of pack_int2_block."""
    buf = np.asarray(buf, np.uint8)
    ng = d // group
    nc = PAGE * d // 4
    nsz = PAGE * ng * scale_bits // 4
    mt = np.float16 if scale_bits == 16 else np.uint8
    kb = buf[:nc].reshape(PAGE, d // 4)
    kf = np.zeros((PAGE, d), np.uint8)
    for m in range(4):
        kf[:, m::4] = (kb >> (2 * m)) & 3
    kc = np.zeros((PAGE, d), np.uint8)
    kc[:, k_code_channel(d, group)] = kf
    o = nc
    ksz = buf[o:o + nsz].copy().view(mt).reshape(PAGE, ng, 2).transpose(1, 0, 2)
    o += nsz
    vb = buf[o:o + nc].reshape(4, d)
    vc = np.zeros((PAGE, d), np.uint8)
    for q in range(4):
        for i in range(4):
            vc[4 * q + i] = (vb[q] >> (2 * i)) & 3
    o += nc
    vsz = buf[o:o + nsz].copy().view(mt).reshape(ng, PAGE, 2)
    return kc, ksz[:, :, 0].T, ksz[:, :, 1].T, vc, vsz[:, :, 0].T, vsz[:, :, 1].T


def pack_bf16_block(k_bits: np.ndarray, v_bits: np.ndarray) -> np.ndarray:
    """k_bits, v_bits: [16, d] bf16 bit patterns -> uint8 block."""
    k = np.asarray(k_bits, np.uint16)
    v = np.asarray(v_bits, np.uint16)
    return np.concatenate([k.view(np.uint8).ravel(), np.ascontiguousarray(v.T).view(np.uint8).ravel()])


# ---------------------------------------------------------------------------
# Where each position lives (logical page, slot) and what an append moves.
# A reference model of the region rule for checking the host planner.
# ---------------------------------------------------------------------------

def bf16_logical_slot(p: int, sink: int, recent: int) -> int:
    """Logical bf16 slot of position p: sink positions keep slot p; recent
    positions use a ring of `recent` slots placed after the sink pages."""
    sink_pages = -(-sink // PAGE)
    if p < sink:
        return p
    return sink_pages * PAGE + (p - sink) % recent


def plan_append(t_old: int, n_new: int, sink: int, recent: int):
    """Moves needed to grow a request from t_old to t_old + n_new tokens.
    Returns (int2_dst, bf16_dst, age_out) where int2_dst[i] / bf16_dst[i] is
    the INT2 position / logical bf16 slot of new token i (or -1), and
    age_out lists (logical bf16 slot, INT2 position) pairs for tokens that
    leave the recent window; those moves come before the new writes."""
    t_new = t_old + n_new
    old = regions(t_old, sink, recent) if t_old else np.zeros(0, np.int8)
    new = regions(t_new, sink, recent)
    age = [(bf16_logical_slot(p, sink, recent), p) for p in range(t_old)
           if old[p] == REGION_RECENT and new[p] == REGION_INT2]
    int2_dst, bf16_dst = [], []
    for i in range(n_new):
        p = t_old + i
        if new[p] == REGION_INT2:
            int2_dst.append(p)
            bf16_dst.append(-1)
        else:
            int2_dst.append(-1)
            bf16_dst.append(bf16_logical_slot(p, sink, recent))
    return np.array(int2_dst, np.int64), np.array(bf16_dst, np.int64), age
