"""Pins of the oracle's calibration against what the pages and mathematics fix:
the composite rotation's closed form, the clip threshold's quantile and its
pooling over a layer, and the grouping of query heads per KV head.

[ES] "Lo que OSCAR hace diferente": R = U H_Had P_br with U the eigenbasis of
the covariance, Lemma 1 and the bit-reversal paragraph.  [IT] 2.2.A: the
per-layer percentile clip threshold taken on the rotated calibration
activations; C_Q and C_S per KV head.

Every expected value here is built by loops or library routines written in
this file, never by the oracle function under test.  Each test also shows
that the slip it targets (P_br dropped, tau from one KV head, the signed
values, the fp64 rotation, the wrong query heads) gives a different value.
"""
import math

import numpy as np
import pytest

import oracle as O


def _rev(k: int, bits: int) -> int:
    """Bit reversal by string reversal (independent of the oracle's helper)."""
    return int(format(k, f"0{bits}b")[::-1], 2)


def _had(a: int, b: int, d: int) -> float:
    """Sylvester Walsh-Hadamard entry, orthonormal."""
    return (-1.0) ** bin(a & b).count("1") / math.sqrt(d)


def _had_matrix(d: int) -> np.ndarray:
    return np.array([[_had(a, b, d) for b in range(d)] for a in range(d)])


def _rand_orth(rng, d):
    a = rng.standard_normal((d, d))
    qm, r = np.linalg.qr(a)
    return qm * np.sign(np.diag(r))


def _closed_form(lam_desc: np.ndarray, permute: bool) -> np.ndarray:
    """R^T C R for R = U H P_br and U the descending eigenbasis of C:
    R^T C R = P^T H (U^T C U) H P = P^T H diag(lam) H P, and since P is
    symmetric and commutes with H this is H diag(lam_rev(k)) H.  Without
    P_br it would be H diag(lam) H."""
    d = lam_desc.size
    bits = d.bit_length() - 1
    mu = np.array([lam_desc[_rev(k, bits)] if permute else lam_desc[k] for k in range(d)])
    h = _had_matrix(d)
    return h @ np.diag(mu) @ h


# --- the composite R = U H P_br by its closed form ---------------------------

@pytest.mark.parametrize("d", [8, 16, 128])
def test_composite_rotation_closed_form(d):
    rng = np.random.default_rng(900 + d)
    o = _rand_orth(rng, d)
    lam = np.sort(rng.exponential(size=d) + 0.05)[::-1]
    c = o @ np.diag(lam) @ o.T
    lam_lib = np.sort(np.linalg.eigvalsh(c))[::-1]
    _, u = O.eig_desc(c)
    r = O.composite_rotation(u)
    got = r.T @ c @ r
    exp = _closed_form(lam_lib, permute=True)
    scale = lam_lib[0]
    assert np.abs(got - exp).max() <= 1e-12 * scale * d
    # teeth: the same rotation without P_br (U H) gives another matrix
    wrong = _closed_form(lam_lib, permute=False)
    assert np.abs(wrong - exp).max() > 1e-3 * scale


def test_composite_rotation_closed_form_by_loops():
    """d = 8, every entry of (U H P)^T C (U H P) against the triple sum
    (1/d) sum_k (-1)^{pc(a&k)+pc(k&b)} lam_rev(k) written out."""
    d, bits = 8, 3
    rng = np.random.default_rng(908)
    o = _rand_orth(rng, d)
    lam = np.array([5.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.25, 0.125])
    c = o @ np.diag(lam) @ o.T
    _, u = O.eig_desc(c)
    got = O.composite_rotation(u).T @ c @ O.composite_rotation(u)
    for a in range(d):
        for b in range(d):
            ref = sum((-1.0) ** (bin(a & k).count("1") + bin(k & b).count("1")) * lam[_rev(k, bits)]
                      for k in range(d)) / d
            assert abs(got[a, b] - ref) < 1e-12


def test_calibrated_rotation_diagonalises_to_the_closed_form():
    """The stored fp32 R_K of calibrate_layer, on a KV head with a distinct
    query spectrum, satisfies R^T C_Q R = H diag(lam_rev) H to fp32
    accuracy, with C_Q built here by loops."""
    d, n, g = 8, 64, 1
    rng = np.random.default_rng(77)
    o = _rand_orth(rng, d)
    scales = np.sqrt(np.array([9.0, 5.0, 3.0, 2.0, 1.2, 0.7, 0.3, 0.1]))
    q = (rng.standard_normal((n, g, d)) * scales) @ o.T
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    cal = O.calibrate_layer(q, k, v)
    cq = np.zeros((d, d))
    for t in range(n):
        for a in range(d):
            for b in range(d):
                cq[a, b] += float(q[t, 0, a]) * float(q[t, 0, b])
    cq /= n
    lam = np.sort(np.linalg.eigvalsh(cq))[::-1]
    r = cal.r_k[0].astype(np.float64)
    got = r.T @ cq @ r
    exp = _closed_form(lam, permute=True)
    assert np.abs(got - exp).max() <= 2e-6 * lam[0]
    assert np.abs(_closed_form(lam, permute=False) - exp).max() > 1e-2 * lam[0]


# --- the clip threshold: linear-interpolation quantile, pooled over the layer ---

def _quantile_by_order_statistics(values, c: float) -> float:
    """Linear interpolation between order statistics: with the n values sorted
    x_(0) <= ... <= x_(n-1), h = (n - 1) c, the c-quantile is
    x_(floor h) + (h - floor h)(x_(floor h + 1) - x_(floor h))."""
    xs = sorted(float(x) for x in values)
    h = (len(xs) - 1) * c
    lo = int(math.floor(h))
    if lo + 1 >= len(xs):
        return xs[-1]
    return xs[lo] + (h - lo) * (xs[lo + 1] - xs[lo])


def test_quantile_linear_small_cases():
    # hand-worked: sorted 1..5, h = 4 * 0.92 = 3.68 -> 4 + 0.68
    assert O.quantile_linear(np.array([5.0, 1.0, 4.0, 2.0, 3.0]), 0.92) == pytest.approx(4.68, abs=1e-12)
    # two values: the straight line between them
    assert O.quantile_linear(np.array([10.0, 0.0]), 0.96) == pytest.approx(9.6, abs=1e-12)
    # an odd count at the median is the middle order statistic, exactly
    assert O.quantile_linear(np.array([3.0, -7.0, 2.5]), 0.5) == 2.5
    assert O.quantile_linear(np.array([4.0]), 0.96) == 4.0
    assert O.quantile_linear(np.array([1.0, 2.0, 3.0]), 1.0) == 3.0
    assert O.quantile_linear(np.array([1.0, 2.0, 3.0]), 0.0) == 1.0


@pytest.mark.parametrize("n", [2, 3, 7, 50, 333])
def test_quantile_linear_against_order_statistics(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n) * rng.exponential(size=n)
    for c in (0.0, 0.1, 0.5, 0.92, 0.96, 0.999, 1.0):
        assert O.quantile_linear(x, c) == pytest.approx(_quantile_by_order_statistics(x, c), rel=1e-14, abs=1e-300)


def _abs_rotated_by_loops(x, r32):
    """|x . R[:, j]| for every token, KV head and channel: fp32 R values,
    exact fp64 products, math.fsum sums."""
    n, hkv, d = x.shape
    out = []
    for t in range(n):
        for h in range(hkv):
            rh = r32[h]
            for j in range(d):
                out.append(abs(math.fsum(float(x[t, h, i]) * float(rh[i, j]) for i in range(d))))
    return out


def _tiny_two_head_layer(seed=5, n=24, g=2, d=8):
    """Two KV heads whose K scales differ x10 one way and V scales x10 the
    other, so a threshold from one head alone lands far from the pooled one."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, 2 * g, d)) * np.array([1.0, 2.0, 0.5, 3.0][:2 * g])[None, :, None]
    k = rng.standard_normal((n, 2, d))
    v = rng.standard_normal((n, 2, d))
    k[:, 1] *= 10.0
    v[:, 0] *= 10.0
    return tuple(a.astype(np.float32) for a in (q, k, v))


def test_tau_is_the_quantile_of_abs_rotated_values_over_all_kv_heads():
    q, k, v = _tiny_two_head_layer()
    cal = O.calibrate_layer(q, k, v)
    for x, r, c, tau in ((k, cal.r_k, 0.96, cal.tau_k), (v, cal.r_v, 0.92, cal.tau_v)):
        vals = _abs_rotated_by_loops(x, r)
        exp = np.float32(_quantile_by_order_statistics(vals, c))
        assert tau == exp
        # teeth: one KV head alone, or the signed values, give other thresholds
        for h in range(2):
            one = np.float32(_quantile_by_order_statistics(_abs_rotated_by_loops(x[:, h:h + 1], r[h:h + 1]), c))
            assert abs(float(one) - float(exp)) > 0.05 * float(exp)
        signed = []
        n, hkv, d = x.shape
        for t in range(n):
            for h in range(hkv):
                for j in range(d):
                    signed.append(math.fsum(float(x[t, h, i]) * float(r[h][i, j]) for i in range(d)))
        assert abs(_quantile_by_order_statistics(signed, c) - float(exp)) > 0.05 * float(exp)


def test_tau_uses_the_stored_fp32_rotation():
    """Keys aligned with columns of the fp64 composite rotate to one large
    entry and d - 1 entries that are zero up to fp64 rounding; with the
    stored fp32 R those entries are the fp32 rounding of R (about 1e-8 of the
    large one).  A 0.5 quantile lands among them, so the threshold taken with
    the fp32 R and the one taken with the fp64 R differ by orders of
    magnitude."""
    d, n = 8, 16
    rng = np.random.default_rng(31)
    q = (rng.standard_normal((n, 1, d)) * np.linspace(3.0, 0.2, d)).astype(np.float32)
    _, u = O.eig_desc(O.query_covariance(q))
    r64 = O.composite_rotation(u)
    k2 = np.empty((n, 1, d))
    for t in range(n):
        k2[t, 0] = (1.0 + t) * r64[:, t % d]
    v = rng.standard_normal((n, 1, d))
    cal = O.calibrate_layer(q, k2, v, clip_k=0.5)
    assert np.array_equal(cal.r_k[0], r64.astype(np.float32))
    exp = _quantile_by_order_statistics(_abs_rotated_by_loops(k2, cal.r_k), 0.5)
    alt = _quantile_by_order_statistics(_abs_rotated_by_loops(k2, r64[None]), 0.5)
    assert exp > 1e-9 and alt < 1e-3 * exp
    assert abs(float(cal.tau_k) - exp) <= 1e-6 * exp


# --- KV-head grouping: C_Q and C_S from the KV head's own query heads --------

def _cq_by_loops(q, heads):
    n, _, d = q.shape
    c = [[0.0] * d for _ in range(d)]
    for e in heads:
        for t in range(n):
            for a in range(d):
                for b in range(d):
                    c[a][b] += float(q[t, e, a]) * float(q[t, e, b])
    return np.array(c) / (n * len(heads))


def _cs_by_loops(q, k, v, heads):
    """(1/(N g)) sum over the heads of (S V)^T (S V), S the causal row-softmax
    of q k^T / sqrt(d), all by loops."""
    n, _, d = q.shape
    c = np.zeros((d, d))
    for e in heads:
        o = np.zeros((n, d))
        for i in range(n):
            logit = [sum(float(q[i, e, a]) * float(k[j, a]) for a in range(d)) / math.sqrt(d) for j in range(i + 1)]
            m = max(logit)
            w = [math.exp(x - m) for x in logit]
            z = sum(w)
            for j in range(i + 1):
                for a in range(d):
                    o[i, a] += w[j] / z * float(v[j, a])
        for a in range(d):
            for b in range(d):
                c[a, b] += sum(o[i, a] * o[i, b] for i in range(n))
    return c / (n * len(heads))


def test_kv_head_grouping_uses_consecutive_query_heads():
    """Hq = 4, Hkv = 2: KV head h is read by query heads 2h and 2h + 1 (the
    decode path's h // g).  The query heads get very different covariances,
    so any other grouping (interleaved heads, every head pooled, one head)
    changes the spectra."""
    n, hkv, g, d = 12, 2, 2, 8
    rng = np.random.default_rng(12)
    q = np.empty((n, hkv * g, d))
    for e in range(hkv * g):
        o = _rand_orth(rng, d)
        q[:, e] = (rng.standard_normal((n, d)) * np.geomspace(4.0 ** (e + 1), 0.1, d)) @ o.T
    k = rng.standard_normal((n, hkv, d)) * np.array([1.0, 3.0])[None, :, None]
    v = rng.standard_normal((n, hkv, d)) * np.array([2.0, 0.5])[None, :, None]
    q, k, v = (x.astype(np.float32) for x in (q, k, v))
    cal = O.calibrate_layer(q, k, v)
    for h in range(hkv):
        heads = [g * h + e for e in range(g)]
        cq = _cq_by_loops(q, heads)
        cs = _cs_by_loops(q, k[:, h], v[:, h], heads)
        lq = np.sort(np.linalg.eigvalsh(cq))[::-1]
        ls = np.sort(np.linalg.eigvalsh(cs))[::-1]
        assert np.allclose(cal.eig_k[h], lq, rtol=1e-10, atol=1e-12 * lq[0])
        assert np.allclose(cal.eig_v[h], ls, rtol=1e-9, atol=1e-12 * ls[0])
        r = cal.r_k[h].astype(np.float64)
        assert np.abs(r.T @ cq @ r - _closed_form(lq, True)).max() <= 2e-6 * lq[0]
        r = cal.r_v[h].astype(np.float64)
        assert np.abs(r.T @ cs @ r - _closed_form(ls, True)).max() <= 2e-6 * ls[0]
        # teeth: the interleaved grouping (heads h, h + Hkv) has another spectrum
        other = [h + hkv * e for e in range(g)]
        lo = np.sort(np.linalg.eigvalsh(_cq_by_loops(q, other)))[::-1]
        assert np.abs(lo - lq).max() > 1e-2 * lq[0]
