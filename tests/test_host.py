"""Host-side checks of liboscar.so that need no GPU: the exported C ABI,
argument validation, offline calibration against the oracle, and the page
pool / region planner against the oracle's reference model of the region rule."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import kv_cache_int2_amd as K
import oracle as O
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        pytest.fail("liboscar.so not built (run __graft_entry__.build())")
    return K.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "oscar.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    declared = set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 20
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(K.EXPORTED), declared ^ set(K.EXPORTED)


def test_block_sizes(lib):
    assert K.oscar_int2_block_bytes(K.make_shape(group=32)) == O.int2_block_bytes(128, 32) == 1536
    assert K.oscar_int2_block_bytes(K.make_shape(group=64)) == O.int2_block_bytes(128, 64) == 1280
    assert K.oscar_bf16_block_bytes(K.make_shape()) == O.bf16_block_bytes(128) == 8192


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), K.OSCAR_EUNSUPPORTED),
    (dict(group=16), K.OSCAR_EUNSUPPORTED),
    (dict(page_size=32), K.OSCAR_EUNSUPPORTED),
    (dict(n_q_heads=3, n_kv_heads=2), K.OSCAR_EINVAL),
    (dict(n_q_heads=64, n_kv_heads=2), K.OSCAR_EUNSUPPORTED),
    (dict(recent=100), K.OSCAR_EUNSUPPORTED),
    (dict(sink=-1), K.OSCAR_EINVAL),
])
def test_shape_validation(lib, kw, code):
    sh = K.make_shape(**kw)
    h = C.c_void_p()
    assert lib.oscar_pool_create(C.byref(sh), 4, 4, C.byref(h)) == code
    assert lib.oscar_last_error()


def test_launch_argument_errors_before_any_gpu_call(lib):
    sh = K.make_shape()
    cache = K.make_cache()
    lay = K.Layer(None, None, 1.0, 1.0)
    # n == 0 is a no-op even without storage
    assert lib.oscar_quant_write(C.byref(sh), C.byref(lay), C.byref(cache), None, None, None, 0, None) == K.OSCAR_OK
    assert lib.oscar_quant_write(C.byref(sh), C.byref(lay), C.byref(cache), None, None, None, 5, None) == K.OSCAR_EINVAL
    assert lib.oscar_quant_write(C.byref(sh), C.byref(lay), C.byref(cache), None, None, None, -1, None) == K.OSCAR_EINVAL
    assert lib.oscar_bf16_write(C.byref(sh), C.byref(cache), None, None, None, 3, None) == K.OSCAR_EINVAL
    assert lib.oscar_copy_pages(C.byref(sh), C.byref(cache), 2, None, None, 1, None) == K.OSCAR_EINVAL
    assert lib.oscar_decode_attn(C.byref(sh), C.byref(lay), C.byref(cache), None, 1, None, 1, None, 1, None, 0, 0,
                                 None, None, 0, None) == K.OSCAR_EINVAL
    assert lib.oscar_decode_attn(C.byref(sh), C.byref(lay), C.byref(cache), None, 0, None, 1, None, 1, None, 0, 0,
                                 None, None, 0, None) == K.OSCAR_OK
    # misaligned storage is refused
    bad = K.Cache(0x1010, 4, 0x2000, 4)
    good_layer = K.Layer(0x1000, 0x2000, 1.0, 1.0)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(good_layer), C.byref(bad), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    nan_layer = K.Layer(0x1000, 0x2000, float("nan"), 1.0)
    ok_cache = K.Cache(0x1000, 4, 0x2000, 4)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(nan_layer), C.byref(ok_cache), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    # an infinite threshold, or one past the largest fp16 with fp16 scale and zero, could
    # overflow s or z; FP8 scale and zero saturate, so 1e5 is accepted there
    for tk, tv in ((float("inf"), 1.0), (1.0, float("-inf")), (65600.0, 1.0), (1.0, 1e6)):
        lay_bad = K.Layer(0x1000, 0x2000, tk, tv)
        assert lib.oscar_quant_write(C.byref(sh), C.byref(lay_bad), C.byref(ok_cache), 0x10, 0x10, 0x10, 1,
                                     None) == K.OSCAR_EINVAL
        assert b"thresholds" in lib.oscar_last_error()
    sh8 = K.make_shape(group=64, scale_bits=8)
    big = K.Layer(0x1000, 0x2000, 1e5, 1e5)
    bad_ptr_cache = K.Cache(0x1010, 4, 0x2000, 4)
    assert lib.oscar_quant_write(C.byref(sh8), C.byref(big), C.byref(bad_ptr_cache), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    assert b"thresholds" not in lib.oscar_last_error()
    # R_K is required; R_V may be NULL (folded into the model's projections), and when given it
    # must be aligned.  The layer passes its check when only R_V is missing: the error is the cache's.
    no_rk = K.Layer(None, 0x2000, 1.0, 1.0)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(no_rk), C.byref(ok_cache), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    assert b"R_K" in lib.oscar_last_error()
    odd_rv = K.Layer(0x1000, 0x2008, 1.0, 1.0)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(odd_rv), C.byref(ok_cache), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    assert b"aligned" in lib.oscar_last_error()
    folded = K.Layer(0x1000, None, 1.0, 1.0)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(folded), C.byref(bad), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    assert b"storage" in lib.oscar_last_error()
    # K/V rows are read 16 bytes at a time
    for kp, vp in ((0x18, 0x10), (0x10, 0x12)):
        assert lib.oscar_quant_write(C.byref(sh), C.byref(good_layer), C.byref(ok_cache), kp, vp, 0x10, 1,
                                     None) == K.OSCAR_EINVAL
        assert b"16-byte" in lib.oscar_last_error()
    # R's prepared digits: n_kv x 2 matrices of 82176 bytes; the buffer must be
    # given, 256-byte aligned and large enough, and a layer's r_prep aligned
    assert K.oscar_layer_prep_bytes(sh) == sh.n_kv_heads * 2 * 82176
    assert K.oscar_layer_prep_bytes(K.make_shape(n_kv_heads=8, n_q_heads=32)) == 16 * 82176
    need = K.oscar_layer_prep_bytes(sh)
    for prep, nbytes in ((None, need), (0x1010, need), (0x1000, need - 1)):
        assert lib.oscar_layer_prepare(C.byref(sh), C.byref(good_layer), prep, nbytes, None) == K.OSCAR_EINVAL
    assert lib.oscar_layer_prepare(C.byref(sh), C.byref(no_rk), 0x1000, need, None) == K.OSCAR_EINVAL
    odd_prep = K.Layer(0x1000, 0x2000, 1.0, 1.0, 0x3010)
    assert lib.oscar_quant_write(C.byref(sh), C.byref(odd_prep), C.byref(ok_cache), 0x10, 0x10, 0x10, 1,
                                 None) == K.OSCAR_EINVAL
    assert b"prepared" in lib.oscar_last_error()
    # the host-table step carries its tables in the launch arguments: at most 64
    # requests, and its host arrays are required
    slots = np.full((4, 65), -1, np.int32)
    ctx = np.ones(65, np.int32)
    assert lib.oscar_decode_step_host_tables(C.byref(sh), C.byref(good_layer), C.byref(ok_cache), 0x10, 0x10,
                                             slots.ctypes.data, 0x10, 65, 0x10, 1, 0x10, 1, ctx.ctypes.data, 0, 0,
                                             0x10, 0x100, 1 << 20, None) == K.OSCAR_EINVAL
    assert b"launch arguments" in lib.oscar_last_error()
    assert lib.oscar_decode_step_host_tables(C.byref(sh), C.byref(good_layer), C.byref(ok_cache), 0x10, 0x10,
                                             None, 0x10, 2, 0x10, 1, 0x10, 1, ctx.ctypes.data, 0, 0, 0x10, 0x100,
                                             1 << 20, None) == K.OSCAR_EINVAL
    assert lib.oscar_decode_step_host_tables(C.byref(sh), C.byref(good_layer), C.byref(ok_cache), 0x10, 0x10,
                                             slots.ctypes.data, 0x10, 0, 0x10, 1, 0x10, 1, ctx.ctypes.data, 0, 0,
                                             0x10, 0x100, 1 << 20, None) == K.OSCAR_OK


def test_workspace_bytes_monotone(lib):
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8)
    a = K.oscar_decode_workspace_bytes(sh, 28, 8, 1)
    b = K.oscar_decode_workspace_bytes(sh, 28, 16, 1)
    assert 0 < a < b and a % 256 == 0
    assert K.oscar_decode_workspace_bytes(sh, 28, 0, 0) >= b
    s = K.oscar_decode_auto_splits(sh, 28, 6300)
    assert 1 <= s <= 128
    assert K.oscar_decode_auto_splits(sh, 1, 64) == 4          # at least 16 pages per split
    assert K.oscar_decode_auto_splits(sh, 1, 2048) == 128      # one 32K-token request: 128 splits
    assert K.oscar_decode_auto_splits(sh, 1, 40000) == 252     # the small-grid form's fit for 8 pairs
    prev = K.oscar_decode_set_small_grid(1)
    try:
        assert K.oscar_decode_auto_splits(sh, 1, 40000) == 128  # capped in the standard form
    finally:
        K.oscar_decode_set_small_grid(prev)
    assert K.oscar_decode_auto_splits(sh, 28, 6300) == 36      # 2 rounds of 4096 wavefronts over 224 (request, head)
    assert K.oscar_decode_auto_splits(sh, 4096, 6300) == 1     # more than two rounds of pairs
    # 12 query heads per KV head at G = 32: three tiles padded to four, one wide wavefront per
    # item, two per SIMD: 2048 at once, two rounds over 16 x 8 pairs = 32 splits
    wide = K.make_shape(n_q_heads=96, n_kv_heads=8, group=32, sink=4, recent=128)
    assert K.oscar_decode_auto_splits(wide, 16, 8200) == 32
    # 8 query heads per KV head: two tiles on one wavefront, three per SIMD: 3072 at once, two
    # rounds over 64 x 8 pairs = 12 splits
    mid = K.make_shape(n_q_heads=64, n_kv_heads=8, group=32, sink=4, recent=128)
    assert K.oscar_decode_auto_splits(mid, 64, 2100) == 12


def test_auto_splits_fit_the_small_grid_form(lib):
    """With the small-grid form allowed (mode 0 or 2) and one-wavefront items,
    the automatic count fits the INT2 items and four bf16 splits into two
    wavefronts per SIMD (2048 on 256 compute units) when that leaves at least
    24 splits; with the form off (mode 1) it is the two-round count."""
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=4, recent=128)
    prev = K.oscar_decode_set_small_grid(0)
    try:
        for mode in (0, 2):
            K.oscar_decode_set_small_grid(mode)
            assert K.oscar_decode_auto_splits(sh, 1, 2048) == 128    # 8 x 132 = 1056 wavefronts fit
            assert K.oscar_decode_auto_splits(sh, 2, 2048) == 124    # 16 x (124 + 4) = 2048
            assert K.oscar_decode_auto_splits(sh, 4, 2048) == 60
            assert K.oscar_decode_auto_splits(sh, 8, 2048) == 28
            assert K.oscar_decode_auto_splits(sh, 9, 2048) == 24     # 2048 // 72 - 4
            assert K.oscar_decode_auto_splits(sh, 10, 2048) == 102   # 21 would be too few: two rounds
            assert K.oscar_decode_auto_splits(sh, 28, 6300) == 36
            # long requests: the whole fit (2048 // 8 - 4) when each of its splits keeps 24 pages
            assert K.oscar_decode_auto_splits(sh, 1, 6250) == 252    # 100K tokens: 24.8 pages a split
            assert K.oscar_decode_auto_splits(sh, 1, 4096) == 128    # 64K tokens: 16.3 at the fit
            assert K.oscar_decode_auto_splits(sh, 2, 6250) == 124    # the fit
            # the workspace for splits 0 covers the largest automatic count (8 pairs: 2048 // 8 - 1)
            assert K.oscar_decode_workspace_bytes(sh, 1, 0, 4) >= K.oscar_decode_workspace_bytes(sh, 1, 255, 4)
        K.oscar_decode_set_small_grid(1)
        assert K.oscar_decode_auto_splits(sh, 2, 2048) == 128
        assert K.oscar_decode_auto_splits(sh, 8, 2048) == 128
        assert K.oscar_decode_auto_splits(sh, 1, 6250) == 128
    finally:
        K.oscar_decode_set_small_grid(prev)


# ---------------------------------------------------------------------------
# calibration vs oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "qwen3_8b_32k"])
def test_calibration_matches_oracle(lib, name):
    w = synth.WORKLOADS[name]
    q, k, v = synth.calib_layer(w, n=1024 if name != "tiny" else None)
    sh = K.make_shape(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, group=w.group)
    rk, rv, ek, ev, tk, tv = K.oscar_calibrate_host(sh, q, k, v)
    cal = O.calibrate_layer(q, k, v)
    assert np.abs(ek / cal.eig_k - 1).max() < 1e-10
    assert np.abs(ev / cal.eig_v - 1).max() < 1e-10
    # same sign convention -> same rotation up to fp32 rounding of a 1e-13 difference
    assert np.abs(rk - cal.r_k).max() < 1e-7 and np.abs(rv - cal.r_v).max() < 1e-7
    assert np.count_nonzero(rk != cal.r_k) < 1e-3 * rk.size
    assert abs(tk / cal.tau_k - 1) < 1e-6 and abs(tv / cal.tau_v - 1) < 1e-6


@pytest.mark.parametrize("rotation", ["identity", "hadamard"])
def test_calibration_rotation_baselines_match_oracle(lib, rotation):
    """The pages' baselines (no rotation; H P_br alone) from the host calibration
    equal the oracle's: the same fixed R, tau under that R, no eigenvalues."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    q, k, v = synth.calib_layer(w, n=512)
    sh = K.make_shape(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, group=w.group)
    rk, rv, ek, ev, tk, tv = K.oscar_calibrate_host(sh, q, k, v, rotation=rotation)
    cal = O.calibrate_layer(q, k, v, rotation=rotation)
    assert np.array_equal(rk, cal.r_k) and np.array_equal(rv, cal.r_v)
    assert np.all(np.isnan(ek)) and np.all(np.isnan(ev))
    assert abs(tk / cal.tau_k - 1) < 1e-6 and abs(tv / cal.tau_v - 1) < 1e-6


def test_calibration_errors(lib):
    sh = K.make_shape()
    z = np.zeros((4, 1, 128), np.float32)
    with pytest.raises(K.OscarError):
        K.oscar_calibrate_host(sh, z, z, z, clip_pct_k=0.0)
    with pytest.raises(K.OscarError):
        K.oscar_calibrate_host(sh, z, z, z, clip_pct_v=1.5)
    r = np.empty((1, 128, 128), np.float32)
    t = C.c_float()
    assert K.lib().oscar_calibrate_host_rotation(C.byref(sh), 7, 4, z.ctypes.data, z.ctypes.data, z.ctypes.data,
                                                 0.96, 0.92, r.ctypes.data, r.ctypes.data, None, None,
                                                 C.addressof(t), C.addressof(t)) == K.OSCAR_EINVAL


# ---------------------------------------------------------------------------
# pools, sequences, planner
# ---------------------------------------------------------------------------

def _phys_to_logical(seq_tables, slot, kind):
    """Map a physical slot back to (logical page, slot) through a block table row."""
    page, s = divmod(int(slot), 16)
    row = seq_tables[kind]
    lp = list(row).index(page)
    return lp * 16 + s


@pytest.mark.parametrize("s0,w", [(4, 128), (64, 256), (0, 16), (5, 32), (4, 0)])
def test_planner_matches_region_model(lib, s0, w):
    sh = K.make_shape(sink=s0, recent=w)
    pool = K.Pool(sh, 400, 40)
    seq = K.oscar_seq_create(pool)
    rng = np.random.default_rng(s0 * 7 + w)
    t = 0
    while t < 1500:
        n = int(min(1500 - t, rng.choice([1, 1, 3, 16, 40, 200])))
        i2, bf, a_s, a_d = K.oscar_seq_plan_append(pool, seq, n)
        r_i2, r_bf, r_age = O.plan_append(t, n, s0, w)
        tables = K.oscar_block_tables(pool, [seq], 200, 40)
        rows = (tables[0][0], tables[1][0])
        assert tables[2][0] == t + n == K.oscar_seq_length(seq)
        for j in range(n):
            if r_i2[j] >= 0:
                assert i2[j] >= 0 and bf[j] == -1
                assert _phys_to_logical(rows, i2[j], 0) == r_i2[j]
            else:
                assert i2[j] == -1 and bf[j] >= 0
                assert _phys_to_logical(rows, bf[j], 1) == r_bf[j]
        assert len(a_s) == len(r_age)
        for (src, dst), (rs, rd) in zip(zip(a_s, a_d), r_age):
            assert _phys_to_logical(rows, src, 1) == rs
            assert _phys_to_logical(rows, dst, 0) == rd
        t += n
    # pages were allocated once each and return on release
    used = 400 - pool.free_pages()[0]
    last_int2 = 1500 - w - 1                             # INT2 positions are [s0, T - w)
    assert used == (last_int2 // 16 - s0 // 16 + 1 if last_int2 >= s0 else 0)
    K.oscar_seq_release(pool, seq)
    assert pool.free_pages() == (400, 40)


def test_pool_exhaustion_leaves_state_unchanged(lib):
    sh = K.make_shape(sink=4, recent=16)
    pool = K.Pool(sh, 3, 2)
    seq = K.oscar_seq_create(pool)
    K.oscar_seq_plan_append(pool, seq, 40)
    before = pool.free_pages()
    with pytest.raises(K.OscarError) as e:
        K.oscar_seq_plan_append(pool, seq, 200)
    assert e.value.code == K.OSCAR_ENOMEM
    assert pool.free_pages() == before and K.oscar_seq_length(seq) == 40
    tables = K.oscar_block_tables(pool, [seq], 8, 8)
    with pytest.raises(K.OscarError):
        K.oscar_block_tables(pool, [seq], 1, 8)         # row too narrow
    assert tables[2][0] == 40


def test_fork_shares_complete_pages_and_copies_open_ones(lib):
    s0, w = 4, 32
    sh = K.make_shape(sink=s0, recent=w)
    pool = K.Pool(sh, 100, 20)
    parent = K.oscar_seq_create(pool)
    K.oscar_seq_plan_append(pool, parent, 100)          # INT2 positions 4..67, ring holds 68..99
    child, src, dst, kind = K.oscar_seq_fork(pool, parent)
    assert K.oscar_seq_length(child) == 100
    pt = K.oscar_block_tables(pool, [parent, child], 16, 8)
    p_i2, c_i2 = pt[0][0], pt[0][1]
    # INT2 pages 0..3 (positions 0..63) are complete -> shared; page 4 (64..79) is open -> copied
    assert list(p_i2[:4]) == list(c_i2[:4])
    assert p_i2[4] != c_i2[4] and p_i2[4] >= 0
    p_bf, c_bf = pt[1][0], pt[1][1]
    assert p_bf[0] == c_bf[0]                            # full sink page shared
    assert p_bf[1] != c_bf[1] and p_bf[2] != c_bf[2]     # ring pages copied
    assert sorted(zip(kind, src, dst)) == sorted(
        [(0, p_i2[4], c_i2[4]), (1, p_bf[1], c_bf[1]), (1, p_bf[2], c_bf[2])])
    # both sequences grow independently; releasing one keeps shared pages alive
    K.oscar_seq_plan_append(pool, child, 50)
    K.oscar_seq_release(pool, parent)
    t = K.oscar_block_tables(pool, [child], 16, 8)
    assert list(t[0][0][:4]) == list(c_i2[:4])
    K.oscar_seq_release(pool, child)
    assert pool.free_pages() == (100, 20)


def test_prefill_auto_splits_fill_the_last_round(lib):
    """With 256 compute units (the host default) and 28 x 8 (request, KV head)
    pairs.  G = 32: a 16-query block (16 tiles) is one item of four wide
    wavefronts, two per SIMD, so 512 run at once; 9 splits fill 2016 of 2048
    (8 would leave the fourth round half empty).  One query (4 tiles) is one
    wide wavefront, 2048 at once: 9 splits again.  G = 64: a 16-query block is
    8 tiles of 8 heads, one 8-wavefront item at four per SIMD, 512 at once: 9
    splits.  Short requests cap the count at one split per 32 pages."""
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=4, recent=128)
    assert K.oscar_prefill_auto_splits(sh, 28, 6300, 128) == 9
    assert K.oscar_prefill_auto_splits(sh, 28, 6300, 1) == 9
    assert K.oscar_prefill_auto_splits(sh, 3, 100, 128) == 3
    assert K.oscar_prefill_auto_splits(sh, 0, 100, 128) == 1
    sh64 = K.make_shape(n_q_heads=32, n_kv_heads=8, group=64, sink=4, recent=128)
    assert K.oscar_prefill_auto_splits(sh64, 28, 6300, 128) == 9


def test_decode_form_setter(lib):
    """oscar_decode_set_small_grid: returns the previous mode, rejects modes
    outside 0..2 with -1 and leaves the mode unchanged."""
    prev = K.oscar_decode_set_small_grid(2)
    try:
        assert prev in (0, 1, 2)
        assert K.oscar_decode_set_small_grid(1) == 2
        assert K.oscar_decode_set_small_grid(3) == -1
        assert K.oscar_decode_set_small_grid(-1) == -1
        assert K.oscar_decode_set_small_grid(0) == 1
        assert K.oscar_decode_set_small_grid(0) == 0
    finally:
        K.oscar_decode_set_small_grid(prev)


def test_prefill_argument_checks(lib):
    """Chunked prefill needs chunk >= 1 and its other arguments (a chunk longer
    than the recent window is accepted); the workspace size grows with the
    chunk up to one query block."""
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=4, recent=128)
    assert K.lib().oscar_prefill_attn(C.byref(sh), None, None, None, 2, 129, None, 1, None, 1, None, 0, 0, None,
                                      None, 0, None) == K.OSCAR_EINVAL
    assert K.lib().oscar_prefill_attn(C.byref(sh), None, None, None, 2, 0, None, 1, None, 1, None, 0, 0, None,
                                      None, 0, None) == K.OSCAR_EINVAL
    a = K.oscar_prefill_workspace_bytes(sh, 28, 1, 8, 1)
    b = K.oscar_prefill_workspace_bytes(sh, 28, 16, 8, 1)
    assert 0 < a < b == K.oscar_prefill_workspace_bytes(sh, 28, 128, 8, 1) == K.oscar_prefill_workspace_bytes(
        sh, 28, 8192, 8, 1)
