"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

  * stored pages: INT2 codes, fp16 scale/zero and bf16 blocks bit-exact;
  * decode attention: max-abs <= 2e-3 and relative-L2 <= 1e-3 against exact
    fp64 attention over the identical stored cache;
  * the all-bf16 baseline decode against exact fp64 attention.
Inputs are the seeded synthetic workloads; the calibration (R, tau) fed to
both sides is the oracle's.
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_int2_amd as K
import oracle as O
import synth
from kv_cache_int2_amd.torch_cache import BaselineCache, DeviceCache

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 2e-3, 1e-3

# decode launch forms (oscar_decode_set_small_grid): 1 one combine work group per
# (request, KV head); 2 the small-grid form (bf16 splits inside the INT2
# kernel's grid, one combine work group per query head) wherever it applies
FORMS = ((1, "standard"), (2, "small-grid"))


class _decode_form:
    def __init__(self, mode):
        self.mode = mode

    def __enter__(self):
        self.prev = K.oscar_decode_set_small_grid(self.mode)
        assert self.prev in (0, 1, 2)

    def __exit__(self, *exc):
        K.oscar_decode_set_small_grid(self.prev)


def _flush(msg):
    print(msg, flush=True)


def _check_close(out, ref, label):
    out = np.asarray(out, np.float64)
    err = np.abs(out - ref).max()
    rel = np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-30)
    _flush(f"{label}: max_abs={err:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(out)), label
    assert err <= MAX_ABS and rel <= REL_L2, (label, err, rel)


def _calibrate(w, hkv=None):
    q, k, v = synth.calib_layer(w)
    if hkv is not None:
        q, k, v = q[:, :hkv * w.gqa], k[:, :hkv], v[:, :hkv]
    return O.calibrate_layer(q, k, v)


def _expected_int2_block(st, lp, h, group):
    t = st.region.shape[0]
    kc = np.zeros((16, 128), np.uint8)
    vc = np.zeros_like(kc)
    ng = 128 // group
    ks, kz, vs, vz = (np.zeros((16, ng), st.k_s.dtype) for _ in range(4))
    for s in range(16):
        p = lp * 16 + s
        if p < t and st.region[p] == O.REGION_INT2:
            kc[s], ks[s], kz[s] = st.k_codes[p, h], st.k_s[p, h], st.k_z[p, h]
            vc[s], vs[s], vz[s] = st.v_codes[p, h], st.v_s[p, h], st.v_z[p, h]
    return O.pack_int2_block(kc, ks, kz, vc, vs, vz)


def _expected_bf16_block(st, lp, h, sink, recent):
    t = st.region.shape[0]
    sp = -(-sink // 16)
    kb = np.zeros((16, 128), np.uint16)
    vb = np.zeros_like(kb)
    for s in range(16):
        pos = None
        if lp < sp:
            if lp * 16 + s < min(sink, t):
                pos = lp * 16 + s
        else:
            r = (lp - sp) * 16 + s
            live = [p for p in range(max(sink, t - recent), t) if (p - sink) % recent == r]
            pos = live[0] if live else None
        if pos is not None:
            kb[s], vb[s] = st.k_bf16[pos, h], st.v_bf16[pos, h]
    return O.pack_bf16_block(kb, vb)


def _check_pages(dc, seq, st, w, label, heads=None):
    i2, bf, ctx = dc.tables([seq])
    heads = range(w.n_kv_heads) if heads is None else heads
    t = int(ctx[0])
    n_int2_pages = 0
    mism = 0
    for lp in range(i2.shape[1]):
        if i2[0, lp] < 0:
            continue
        n_int2_pages += 1
        for h in heads:
            got = dc.int2_block_bytes_of(int(i2[0, lp]), h)
            exp = _expected_int2_block(st, lp, h, w.group)
            if not np.array_equal(got, exp):
                mism += 1
                if mism < 4:
                    bad = np.nonzero(got != exp)[0]
                    _flush(f"{label}: INT2 page {lp} head {h}: {bad.size} bytes differ, first at {bad[:8]}")
    for lp in range(bf.shape[1]):
        if bf[0, lp] < 0:
            continue
        for h in heads:
            got = dc.bf16_block_bytes_of(int(bf[0, lp]), h)
            exp = _expected_bf16_block(st, lp, h, w.sink, w.recent)
            if not np.array_equal(got, exp):
                mism += 1
                _flush(f"{label}: bf16 page {lp} head {h} differs")
    _flush(f"{label}: T={t} int2 pages={n_int2_pages} mismatching blocks={mism}")
    assert mism == 0


def _fill(dc, seq, kb, vb, plan):
    """plan: list of chunk sizes summing to len(kb)."""
    t = 0
    for n in plan:
        dc.append(seq, kb[t:t + n], vb[t:t + n])
        t += n
    assert t == kb.shape[0]


# ---------------------------------------------------------------------------

def test_tiny_write_pages_and_decode():
    w = synth.WORKLOADS["tiny"]
    _flush("case tiny: T=4096 Hq=Hkv=1 G=32")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=1, n_kv_heads=1, group=32, sink=w.sink, recent=w.recent)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 300, 16)
    kb, vb = synth.kv_request_bf16(w, 0, 0, w.context)
    seq = dc.new_seq()
    # prefill in uneven chunks, then single-token decode steps (ring age-out path)
    _fill(dc, seq, kb, vb, [1000, 1, 2000, 77, 999] + [1] * 19)
    st = O.store_request(kb, vb, cal, w.group, w.sink, w.recent)
    _check_pages(dc, seq, st, w, "tiny")
    q = synth.q_decode_bf16(w, 0)[None]
    out = dc.decode([seq], q).cpu().numpy()
    ref = O.decode_attention(q[0], st, cal, w.group)[None]
    _check_close(out, ref, "tiny decode")
    # 200 splits: more splits than some pages hold tokens for (empty partials);
    # fewer than 8 splits leave some of the small-grid combine's merge ranges empty
    for mode, form in FORMS:
        with _decode_form(mode):
            for si in (1, 3, 7, 64, 200):
                out = dc.decode([seq], q, splits_int2=si).cpu().numpy()
                _check_close(out, ref, f"tiny decode {form} splits={si}")


def test_qwen3_8b_layer_32k():
    w = synth.WORKLOADS["qwen3_8b_32k"]
    _flush("case qwen3_8b_32k: T=32768 Hq=32 Hkv=8 G=32")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=w.sink, recent=w.recent)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 2100, 16)
    kb, vb = synth.kv_request_bf16(w, 0, 0, w.context)
    seq = dc.new_seq()
    _fill(dc, seq, kb, vb, [8192, 8192, 8192, 8190, 1, 1])
    st = O.store_request(kb, vb, cal, w.group, w.sink, w.recent)
    _check_pages(dc, seq, st, w, "qwen3_8b_32k")
    q = synth.q_decode_bf16(w, 0)[None]
    ref = O.decode_attention(q[0], st, cal, w.group)[None]
    # past 64 splits the combine merges chunks of 64 partial rows in groups of
    # 16: 100 (a partial group), 128 (two chunks), 130 (a third chunk of two)
    for mode, form in FORMS:
        with _decode_form(mode):
            for si in (0, 5, 16, 100, 128, 130, 256):
                out = dc.decode([seq], q, splits_int2=si).cpu().numpy()
                _check_close(out, ref, f"qwen3_8b_32k decode {form} splits={si}")


@pytest.mark.parametrize("hq,hkv,group,scale_bits", [(4, 1, 32, 16), (8, 1, 32, 16), (12, 1, 32, 16), (16, 1, 32, 16),
                                                      (12, 1, 64, 16), (4, 2, 64, 16), (16, 1, 64, 16),
                                                      (4, 1, 64, 8), (8, 1, 32, 8), (12, 1, 64, 8)])
def test_ragged_batch_gqa_groups(hq, hkv, group, scale_bits):
    """Mixed lengths (all-bf16, exactly sink+recent, one INT2 token, odd page
    counts) in one batch, for several GQA widths, both group sizes and both
    scale/zero formats."""
    w = synth.Workload("ragged", 10 + hq + group, hq, hkv, 128, 1, 0, group=group, sink=4, recent=32,
                       outlier_scale=(40.0, 40.0), calib_tokens=512)
    _flush(f"case ragged hq={hq} hkv={hkv} G={group} scale_bits={scale_bits}")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=group, sink=4, recent=32, scale_bits=scale_bits)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 600, 64)
    lens = [1, 5, 36, 37, 53, 100, 515, 1000, 2049, 3001]
    seqs, stores, qs = [], [], []
    for r, t in enumerate(lens):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        seq = dc.new_seq()
        _fill(dc, seq, kb, vb, [t] if t < 200 else [t - 7] + [1] * 7)
        seqs.append(seq)
        stores.append(O.store_request(kb, vb, cal, group, 4, 32, scale_bits))
        qs.append(synth.q_decode_bf16(w, r))
    for r in (0, 6, 9):
        _check_pages(dc, seqs[r], stores[r], w, f"ragged len={lens[r]}")
    q = np.stack(qs)
    ref = np.stack([O.decode_attention(q[r], stores[r], cal, group) for r in range(len(lens))])
    # bf16 splits <= 4 run inside the combine kernel, 5 in their own kernel
    # (the small-grid form: all inside the INT2 kernel's grid)
    for mode, form in FORMS:
        with _decode_form(mode):
            for si, sb in ((0, 0), (1, 1), (4, 3), (1, 5)):
                out = dc.decode(seqs, q, splits_int2=si, splits_bf16=sb).cpu().numpy()
                for r in range(len(lens)):
                    _check_close(out[r], ref[r], f"ragged {form} hq={hq} G={group} len={lens[r]} splits={si}/{sb}")


@pytest.mark.parametrize("group,scale_bits", [(32, 16), (64, 8)])
def test_unwritten_slots_may_hold_nan(group, scale_bits):
    """Pools that start as all-0xFF bytes (every unwritten bf16 value and
    scale/zero a NaN): the slots no position owns yet (sink page tail, recent
    ring not yet full, the INT2 pages at the region edges) must not reach the
    outputs, in decode and in a chunked prefill longer than the window."""
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    w = synth.Workload("nanfill", 70 + group, 8, 1, 128, 1, 0, group=group, sink=4, recent=32,
                       outlier_scale=(20.0, 20.0), calib_tokens=512)
    _flush(f"case nan-filled pools G={group} scale_bits={scale_bits}")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=8, n_kv_heads=1, group=group, sink=4, recent=32, scale_bits=scale_bits)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 400, 64, fill=0xFF)
    lens = [1, 5, 21, 36, 37, 53, 515, 2049]
    seqs, stores, kvs = [], [], []
    for r, t in enumerate(lens):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        seq = dc.new_seq()
        _fill(dc, seq, kb, vb, [t] if t < 200 else [t - 7] + [1] * 7)
        seqs.append(seq)
        stores.append(O.store_request(kb, vb, cal, group, 4, 32, scale_bits))
    q = np.stack([synth.q_decode_bf16(w, r) for r in range(len(lens))])
    ref = np.stack([O.decode_attention(q[r], stores[r], cal, group) for r in range(len(lens))])
    for mode, form in FORMS:
        with _decode_form(mode):
            for si, sb in ((0, 0), (3, 3), (1, 5)):
                out = dc.decode(seqs, q, splits_int2=si, splits_bf16=sb).cpu().numpy()
                for r in range(len(lens)):
                    _check_close(out[r], ref[r], f"nan-filled {form} G={group} len={lens[r]} splits={si}/{sb}")
    # a chunk of 45 new tokens (past the 32-token window) on two of the requests
    chunk = 45
    pf = [seqs[4], seqs[6]]
    qc = np.stack([np.stack([synth.q_decode_bf16(w, 50 + r, c) for c in range(chunk)]) for r in range(2)])
    pst = []
    for r, (seq, t) in enumerate(((seqs[4], lens[4]), (seqs[6], lens[6]))):
        kb, vb = synth.kv_request_bf16(w, 4 if r == 0 else 6, 0, t + chunk)
        dc.append(seq, kb[t:], vb[t:])
        pst.append(O.store_request(kb, vb, cal, group, 4, 32, scale_bits))
    i2, bf, ctx = dc.tables(pf)
    ws = torch.empty(K.oscar_prefill_workspace_bytes(sh, 2, chunk), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, chunk, 8, 128), dtype=torch.float32, device="cuda")
    K.oscar_prefill_attn(sh, dc.layer, dc.cache, to_dev_bits(qc), to_dev_i32(i2), to_dev_i32(bf), to_dev_i32(ctx),
                         out, ws)
    got = out.cpu().numpy()
    for r in range(2):
        _check_close(got[r], O.prefill_attention(qc[r], pst[r], cal, group), f"nan-filled prefill {r}")


def test_empty_context_gives_zero_rows():
    w = synth.WORKLOADS["tiny"]
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=1, n_kv_heads=1, group=32)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 8, 16)
    empty = dc.new_seq()
    full = dc.new_seq()
    kb, vb = synth.kv_request_bf16(w, 0, 0, 200)
    dc.append(full, kb, vb)
    q = np.stack([synth.q_decode_bf16(w, 0), synth.q_decode_bf16(w, 1)])
    st = O.store_request(kb, vb, cal, 32, w.sink, w.recent)
    for mode, form in FORMS:
        with _decode_form(mode):
            out = dc.decode([empty, full], q).cpu().numpy()
        assert np.all(out[0] == 0), form
        _check_close(out[1], O.decode_attention(q[1], st, cal, 32), f"after empty row ({form})")


@pytest.mark.parametrize("scale_bits", [16, 8])
def test_quant_write_scattered_slots_and_nan_group(scale_bits):
    """Tokens written in shuffled order into scattered slots (V words merged by
    atomics across wavefronts) and a NaN input row, with fp16 and with FP8
    scale and zero."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=0, recent=0, scale_bits=scale_bits)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 64, 1)
    n = 37 * 16
    kb, vb = synth.kv_request_bf16(w, 3, 0, n)
    kb[100, 2, 5] = 0x7FC0                       # bf16 NaN in K of token 100, head 2
    rng = np.random.default_rng(0)
    slots = rng.permutation(64 * 16)[:n].astype(np.int32)
    order = rng.permutation(n)
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    K.oscar_quant_write(sh, dc.layer, dc.cache, to_dev_bits(kb[order]), to_dev_bits(vb[order]),
                        to_dev_i32(slots[order]))
    torch.cuda.synchronize()
    pool = dc.int2.cpu().numpy().reshape(64, 8, -1)
    for h in (0, 2, 7):
        xk = O.bf16_to_f64(kb[:, h])
        xv = O.bf16_to_f64(vb[:, h])
        ck, sk, zk, _ = O.quantize(xk, cal.r_k[h], cal.tau_k, 32, scale_bits)
        cv, sv, zv, _ = O.quantize(xv, cal.r_v[h], cal.tau_v, 32, scale_bits)
        bits = np.uint16 if scale_bits == 16 else np.uint8
        for i in range(n):
            page, s = divmod(int(slots[i]), 16)
            blk = O.unpack_int2_block(pool[page, h], 128, 32, scale_bits)
            assert np.array_equal(blk[0][s], ck[i]), (h, i)
            assert np.array_equal(blk[3][s], cv[i]), (h, i)
            if h == 2 and i == 100:
                assert np.all(np.isnan(O.meta_values(blk[1][s]))) and np.all(np.isnan(O.meta_values(blk[2][s])))
                continue
            assert np.array_equal(blk[1][s].view(bits), sk[i].view(bits))
            assert np.array_equal(blk[2][s].view(bits), zk[i].view(bits))
            assert np.array_equal(blk[4][s].view(bits), sv[i].view(bits))
            assert np.array_equal(blk[5][s].view(bits), zv[i].view(bits))


def test_shared_prefix_fork():
    """Prefix caching: children forked from one parent share its complete pages
    (same physical ids) and decode like independent requests."""
    w = synth.Workload("prefix", 42, 8, 1, 128, 1, 0, sink=4, recent=32, shared_prefix=4096, calib_tokens=512)
    _flush("case shared prefix fork")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=8, n_kv_heads=1, group=32, sink=4, recent=32)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 2000, 64)
    parent = dc.new_seq()
    pk, pv = synth.kv_request_bf16(w, 0, 0, 4096)   # shared prefix (generator's shared id)
    dc.append(parent, pk, pv)
    kids, stores, qs = [], [], []
    for r in range(4):
        c = dc.fork(parent)
        own_k, own_v = synth.kv_request_bf16(w, r + 1, 4096, 4096 + 700 + 13 * r)
        dc.append(c, own_k[:500], own_v[:500])
        for i in range(500, own_k.shape[0]):
            dc.append(c, own_k[i:i + 1], own_v[i:i + 1])
        kb = np.concatenate([pk, own_k])
        vb = np.concatenate([pv, own_v])
        kids.append(c)
        stores.append(O.store_request(kb, vb, cal, 32, 4, 32))
        qs.append(synth.q_decode_bf16(w, r))
    tabs = dc.tables(kids)
    shared = (4096 - 32) // 16                      # complete INT2 pages at fork time
    for r in range(1, 4):
        assert np.array_equal(tabs[0][r, :shared], tabs[0][0, :shared])
        assert tabs[0][r, shared] != tabs[0][0, shared]
    for r in range(4):
        _check_pages(dc, kids[r], stores[r], w, f"fork child {r}")
    q = np.stack(qs)
    out = dc.decode(kids, q).cpu().numpy()
    for r in range(4):
        _check_close(out[r], O.decode_attention(q[r], stores[r], cal, 32), f"fork child {r} decode")


@pytest.mark.parametrize("hq,hkv", [(1, 1), (32, 8), (12, 1)])
def test_bf16_baseline_decode(hq, hkv):
    w = synth.Workload("base", 50 + hq, hq, hkv, 128, 1, 0, calib_tokens=256)
    _flush(f"case bf16 baseline hq={hq} hkv={hkv}")
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv)
    bc = BaselineCache(sh, 1200, 5000)
    lens = [1, 17, 300, 4999]
    seqs, ks, vs = [], [], []
    for r, t in enumerate(lens):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        s = bc.new_seq()
        bc.append(s, kb, vb)
        seqs.append(s)
        ks.append(kb)
        vs.append(vb)
    q = np.stack([synth.q_decode_bf16(w, r) for r in range(len(lens))])
    for sp in (0, 1, 5):
        out = bc.decode(seqs, q, splits=sp).cpu().numpy()
        for r in range(len(lens)):
            ref = O.attend(O.bf16_to_f64(q[r]), O.bf16_to_f64(ks[r]), O.bf16_to_f64(vs[r]))
            _check_close(out[r], ref, f"baseline hq={hq} len={lens[r]} splits={sp}")


def _full_size_sampled(w, group, check, scale_bits=16):
    """Fill a workload at full size (a shared prefix through a fork, as the
    bench does), decode the whole batch in the bench's launch configuration
    (automatic split count), and check the requests in `check`: every query
    head's output, and a spread of their page blocks, against the oracle run on
    those requests alone."""
    B, T = w.batch, w.context
    _flush(f"case {w.name}: B={B} T={T} Hq={w.n_q_heads} Hkv={w.n_kv_heads} G={group} sink={w.sink} "
           f"recent={w.recent} scale_bits={scale_bits}")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, group=group, sink=w.sink,
                      recent=w.recent, scale_bits=scale_bits)
    ppr = (T + 15) // 16 + 2
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, B * ppr + 8,
                     B * (w.sink // 16 + 2 + w.recent // 16) + 8)
    parent, start = None, 0
    if w.shared_prefix:
        start = w.shared_prefix
        kb, vb = synth.kv_request_bf16(w, 0, 0, start)
        parent = dc.new_seq()
        _fill(dc, parent, kb, vb, [start])
    seqs = []
    for r in range(B):
        kb, vb = synth.kv_request_bf16(w, r, start, T)
        seq = dc.fork(parent) if parent is not None else dc.new_seq()
        n = T - start
        _fill(dc, seq, kb, vb, [16384] * (n // 16384) + ([n % 16384] if n % 16384 else []))
        seqs.append(seq)
    _flush("filled")
    q = np.stack([synth.q_decode_bf16(w, r, 1) for r in range(B)])
    out = dc.decode(seqs, q).cpu().numpy()
    assert np.all(np.isfinite(out))
    i2, bf, _ = dc.tables(seqs)
    for r in check:
        kb, vb = synth.kv_request_bf16(w, r, 0, T)
        st = O.store_request(kb, vb, cal, group, w.sink, w.recent, scale_bits)
        _check_close(out[r], O.decode_attention(q[r], st, cal, group), f"{w.name} G={group} request {r}")
        # page blocks: the first INT2 pages, pages spread over the history, the last ones
        # (logical INT2 pages before the sink's end hold no token and have no block)
        have = np.nonzero(i2[r] >= 0)[0]
        n_lp = have.size
        lps = sorted({int(have[i]) for i in (0, 1, 2, n_lp // 3, n_lp // 2, 2 * n_lp // 3, n_lp - 2, n_lp - 1)})
        mism = 0
        def differ(kind, lp, h, got, exp):
            bad = np.nonzero(got != exp)[0]
            if bad.size:
                _flush(f"{w.name} request {r}: {kind} page {lp} head {h}: {bad.size} bytes differ at "
                       f"{bad[:6].tolist()}: got {got[bad[:6]].tolist()} expected {exp[bad[:6]].tolist()}")
            return int(bad.size > 0)
        for lp in lps:
            for h in range(w.n_kv_heads):
                got = dc.int2_block_bytes_of(int(i2[r, lp]), h)
                mism += differ("INT2", lp, h, got, _expected_int2_block(st, lp, h, group))
            for lpb in range(bf.shape[1]):
                if bf[r, lpb] >= 0 and lp == lps[0]:
                    for h in range(w.n_kv_heads):
                        got = dc.bf16_block_bytes_of(int(bf[r, lpb]), h)
                        mism += differ("bf16", lpb, h, got, _expected_bf16_block(st, lpb, h, w.sink, w.recent))
        _flush(f"{w.name} G={group} request {r}: {len(lps)} INT2 pages x {w.n_kv_heads} heads and the bf16 "
               f"pages, mismatching blocks={mism}")
        assert mism == 0


def test_full_size_28x100k_sampled():
    """The measured workload: 28 requests x 100000 tokens, g = 4."""
    w = synth.WORKLOADS["long_28x100k"]
    _full_size_sampled(w, w.group, (0, w.batch - 1))


def test_full_size_prefix_64x32k_sampled():
    """64 requests x 32768 tokens sharing an 8192-token prefix through the block
    tables, g = 8 (two row tiles on one wavefront)."""
    w = synth.WORKLOADS["qwen3_32b_prefix"]
    _full_size_sampled(w, w.group, (0, w.batch - 1))


def test_full_size_28x100k_pages_layout_sampled():
    """The pages' default layout on the 28 x 100k batch: sink 64, recent 256,
    G = 64 with FP8 scale and zero (2.25 history bits per element)."""
    import dataclasses
    w = dataclasses.replace(synth.WORKLOADS["long_28x100k"], sink=64, recent=256, group=64)
    _full_size_sampled(w, 64, (0, w.batch - 1), scale_bits=8)


@pytest.mark.parametrize("group", [32, 64])
def test_full_size_stress_16x128k_sampled(group):
    """16 requests x 131072 tokens, g = 12, both group sizes (three tiles as
    three wavefronts at G = 32, two tiles on one wavefront at G = 64)."""
    w = synth.WORKLOADS["stress_16x128k"]
    _full_size_sampled(w, group, (w.batch - 1,))


@pytest.mark.parametrize("hq,hkv,group,sink,recent,scale_bits,reps", [
    (8, 2, 32, 4, 32, 16, 1), (12, 1, 64, 20, 48, 16, 1), (4, 1, 32, 4, 0, 16, 1), (4, 2, 64, 64, 48, 8, 1),
    (16, 1, 32, 0, 16, 16, 1), (4, 1, 64, 0, 0, 8, 1),
    # 8 KV heads x 15 and 25 requests: the prologue's step writes in one work
    # group per (request, KV head) (120 pairs) and inside the q-operand work
    # groups (200 pairs); the cases above run one writer per K and V matrix
    (32, 8, 32, 4, 32, 16, 3), (32, 8, 32, 4, 32, 16, 5)])
def test_fused_decode_step(hq, hkv, group, sink, recent, scale_bits, reps):
    """oscar_decode_step (writes fused into the decode's prologue kernel) against
    the separate write calls + oscar_decode_attn: identical cache bytes and bit-identical outputs after every step,
    through ring age-out, page crossings, sink growth and (recent = 0) new
    tokens quantised straight to INT2, with no sink region (sink = 0) and with
    every position INT2 (sink = recent = 0); oscar_decode_step_host_tables (the
    step tables in host memory, carried in the launch arguments) identical to
    oscar_decode_step at every step; then the pages bit-exact and the output
    within tolerance against the oracle."""
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    w = synth.Workload("fused", 70 + hq + group, hq, hkv, 128, 1, 0, group=group, sink=sink, recent=recent,
                       outlier_scale=(40.0, 40.0), calib_tokens=512)
    _flush(f"case fused step hq={hq} hkv={hkv} G={group} sink={sink} recent={recent} scale_bits={scale_bits} "
           f"batch={5 * reps}")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=group, sink=sink, recent=recent, scale_bits=scale_bits)
    lens0 = [0, 3, max(sink + recent - 2, 1), 200, 1001] * reps
    n_steps = 40 if reps == 1 else 20
    B = len(lens0)
    caches = [DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 600 * reps, 64 * reps) for _ in range(3)]
    seqs = [[], [], []]
    for r, t in enumerate(lens0):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        for c in (0, 1, 2):
            s = caches[c].new_seq()
            if t:
                caches[c].append(s, kb, vb)
            seqs[c].append(s)
    planners = [K.DecodeStepPlanner(caches[c].pool, seqs[c]) for c in (0, 1, 2)]
    max_i2 = (max(lens0) + n_steps + 15) // 16
    max_bf = -(-sink // 16) + recent // 16 + 1
    si = 3
    ws = [torch.empty(K.oscar_decode_workspace_bytes(sh, B, si, 1), dtype=torch.uint8, device="cuda")
          for _ in (0, 1, 2)]
    outs = [torch.empty((B, hq, 128), dtype=torch.float32, device="cuda") for _ in (0, 1, 2)]
    for st in range(n_steps):
        kn = np.stack([synth.kv_request_bf16(w, r, lens0[r] + st, lens0[r] + st + 1)[0][0] for r in range(B)])
        vn = np.stack([synth.kv_request_bf16(w, r, lens0[r] + st, lens0[r] + st + 1)[1][0] for r in range(B)])
        q = to_dev_bits(np.stack([synth.q_decode_bf16(w, r, st + 1) for r in range(B)]))
        kd, vd = to_dev_bits(kn), to_dev_bits(vn)
        res = [planners[c].step() for c in (0, 1, 2)]
        bufs = [planners[c].buf.copy() for c in (0, 1, 2)]
        assert np.array_equal(bufs[0], bufs[1]) and np.array_equal(bufs[0], bufs[2]) and res[0] == res[1] == res[2]
        d = to_dev_i32(bufs[0])
        tabs = [caches[c].tables(seqs[c], max_i2, max_bf) for c in (0, 1, 2)]
        dt = [(to_dev_i32(i2), to_dev_i32(bf), to_dev_i32(ctx)) for i2, bf, ctx in tabs]
        c0, c1 = caches[0], caches[1]
        # both launch forms, alternating by step (the three calls of one step
        # take the same form)
        with _decode_form(FORMS[st % 2][0]):
            # separate calls
            if res[0][0]:
                K.oscar_requant_from_bf16(sh, c0.layer, c0.cache, d[2], d[3], n=B)
            if np.any(bufs[0][0] >= 0):
                K.oscar_quant_write(sh, c0.layer, c0.cache, kd, vd, d[0], n=B)
            if np.any(bufs[0][1] >= 0):
                K.oscar_bf16_write(sh, c0.cache, kd, vd, d[1], n=B)
            K.oscar_decode_attn(sh, c0.layer, c0.cache, q, *dt[0][:2], dt[0][2], outs[0], ws[0], si, 1)
            # fused step
            K.oscar_decode_step(sh, c1.layer, c1.cache, kd, vd, d[:4], q, *dt[1][:2], dt[1][2], outs[1], ws[1],
                                si, 1)
            # fused step, tables from host memory (the array is overwritten right
            # after the call: the launch arguments hold their own copy)
            host_tab = bufs[2].copy()
            K.oscar_decode_step_host_tables(sh, caches[2].layer, caches[2].cache, kd, vd, host_tab[:4], q, *dt[2][:2],
                                            host_tab[4], outs[2], ws[2], si, 1)
            host_tab[:] = -7
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {st}: outputs differ"
        assert torch.equal(outs[1], outs[2]), f"step {st}: host-table step differs"
        if st % 8 == 7 or st == n_steps - 1:
            assert torch.equal(c0.int2, c1.int2), f"step {st}: INT2 storage differs"
            assert torch.equal(c0.bf16, c1.bf16), f"step {st}: bf16 storage differs"
            assert torch.equal(c1.int2, caches[2].int2) and torch.equal(c1.bf16, caches[2].bf16), \
                f"step {st}: host-table step storage differs"
    _flush(f"fused step: {n_steps} steps identical to the separate calls")
    out = outs[1].cpu().numpy()
    qf = np.stack([synth.q_decode_bf16(w, r, n_steps) for r in range(B)])
    for r in range(B):
        t = lens0[r] + n_steps
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        store = O.store_request(kb, vb, cal, group, sink, recent, scale_bits)
        _check_pages(caches[1], seqs[1][r], store, w, f"fused step len={t}")
        _check_close(out[r], O.decode_attention(qf[r], store, cal, group), f"fused step decode len={t}")


@pytest.mark.parametrize("rotation", ["oscar", "identity", "hadamard"])
def test_f1_rotation_ablation_through_the_kernels(rotation):
    """The pages' baselines (naive INT2, Hadamard only) run through the same
    write and decode kernels as OSCAR: pages bit-exact and outputs within
    tolerance against the oracle under that rotation; the output error against
    exact attention over the unquantised cache is reported."""
    w = synth.WORKLOADS["qwen3_8b_32k"]
    t = 8192
    _flush(f"case f1 rotation={rotation}: T={t} Hq=32 Hkv=8 G=32")
    q, k, v = synth.calib_layer(w)
    cal = O.calibrate_layer(q, k, v, rotation=rotation)
    sh = K.make_shape(n_q_heads=32, n_kv_heads=8, group=32, sink=w.sink, recent=w.recent)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 600, 16)
    kb, vb = synth.kv_request_bf16(w, 0, 0, t)
    seq = dc.new_seq()
    _fill(dc, seq, kb, vb, [4096, 4000, 1] + [1] * 95)
    st = O.store_request(kb, vb, cal, w.group, w.sink, w.recent)
    _check_pages(dc, seq, st, w, f"f1 {rotation}")
    kx, vx = O.bf16_to_f64(kb), O.bf16_to_f64(vb)
    oe = on = 0.0
    for s in range(4):
        qb = synth.q_decode_bf16(w, 0, s)
        out = dc.decode([seq], qb[None]).cpu().numpy()[0].astype(np.float64)
        _check_close(out, O.decode_attention(qb, st, cal, w.group), f"f1 {rotation} decode {s}")
        ex = O.attend(O.bf16_to_f64(qb), kx, vx)
        oe += float(((out - ex) ** 2).sum())
        on += float((ex ** 2).sum())
    _flush(f"f1 rotation={rotation}: output error vs unquantised cache rel_l2={math.sqrt(oe / on):.4f} "
           f"tau_k={float(cal.tau_k):.3f} tau_v={float(cal.tau_v):.3f}")


@pytest.mark.parametrize("hq,hkv,group,scale_bits,t0,chunk", [
    (32, 8, 32, 16, 3000, 16), (4, 1, 32, 16, 700, 37), (8, 2, 64, 8, 5000, 128),
    (1, 1, 32, 16, 300, 100), (16, 1, 32, 16, 2000, 20), (12, 1, 64, 16, 1500, 7),
    (32, 8, 32, 16, 3000, 300), (8, 2, 64, 8, 500, 1000), (12, 1, 32, 16, 200, 403), (1, 1, 32, 16, 90, 250),
    (4, 1, 32, 16, 500, 3)])
def test_f2_prefill_attention(hq, hkv, group, scale_bits, t0, chunk):
    """Chunked prefill over the mixed cache: a chunk of new tokens is written
    (their entry into the recent window pushes older tokens into INT2), then
    its queries attend causally; every query head of every chunk query against
    the oracle.  Requests of different lengths, one made of the chunk alone,
    several query blocks per launch (g = 4, G = 32: 16 queries a block), and
    chunks longer than the recent window, whose older positions the queries
    read as INT2 up to their own."""
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    w = synth.Workload("prefill", 120 + hq + chunk, hq, hkv, 128, 1, 0, group=group, sink=4, recent=128,
                       outlier_scale=(20.0, 20.0), calib_tokens=512)
    _flush(f"case f2 prefill hq={hq} hkv={hkv} G={group} scale_bits={scale_bits} t0={t0} chunk={chunk}")
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=group, sink=4, recent=128, scale_bits=scale_bits)
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, 1200, 64)
    starts = [t0, t0 // 3 + 11, 0]
    seqs = []
    for r, s0 in enumerate(starts):
        kb, vb = synth.kv_request_bf16(w, r, 0, s0 + chunk)
        seq = dc.new_seq()
        if s0:
            dc.append(seq, kb[:s0], vb[:s0])
        dc.append(seq, kb[s0:], vb[s0:])           # the chunk's own tokens
        seqs.append(seq)
    i2, bf, ctx = dc.tables(seqs)
    q = np.stack([np.stack([synth.q_decode_bf16(w, r, c) for c in range(chunk)]) for r in range(len(starts))])
    B = len(starts)
    ws = torch.empty(K.oscar_prefill_workspace_bytes(sh, B, chunk), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, chunk, hq, 128), dtype=torch.float32, device="cuda")
    K.oscar_prefill_attn(sh, dc.layer, dc.cache, to_dev_bits(q), to_dev_i32(i2), to_dev_i32(bf), to_dev_i32(ctx),
                         out, ws)
    got = out.cpu().numpy()
    for r, s0 in enumerate(starts):
        kb, vb = synth.kv_request_bf16(w, r, 0, s0 + chunk)
        st = O.store_request(kb, vb, cal, group, 4, 128, scale_bits)
        ref = O.prefill_attention(q[r], st, cal, group)
        _check_close(got[r], ref, f"f2 prefill request {r} T={s0 + chunk} chunk={chunk}")


def test_f4_rv_folded_into_the_projections():
    """R_V folded into the model's projections ([ES] serving section): V
    arrives as v R_V (bf16) and the layer has r_v = NULL, so the writes quantise
    it unrotated and the output stays in the rotated basis.  Through the write
    calls and then fused decode steps: storage and outputs bit-identical to
    passing R_V = I, pages bit-exact and outputs within tolerance against the
    oracle with R_V = I on the same folded V, and the output, rotated back,
    as accurate against exact attention as the unfolded path's."""
    import dataclasses
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    hq, hkv, sink, recent = 8, 2, 4, 32
    w = synth.Workload("fold", 77, hq, hkv, 128, 1, 0, group=32, sink=sink, recent=recent,
                       outlier_scale=(20.0, 20.0), calib_tokens=512)
    _flush("case f4 R_V folded")
    cal = _calibrate(w)
    eye = np.broadcast_to(np.eye(128, dtype=np.float32), cal.r_v.shape).copy()
    cal_i = dataclasses.replace(cal, r_v=eye)
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=32, sink=sink, recent=recent)
    r_v64 = cal.r_v.astype(np.float64)

    def folded(vb):  # the folded projection's output, rounded to bf16 as a model would
        return synth.f32_to_bf16_bits(np.einsum("thd,hde->the", O.bf16_to_f64(vb), r_v64).astype(np.float32))

    lens0, n_steps = [3, 37, 600], 24
    B = len(lens0)
    caches = [DeviceCache(sh, cal.r_k, rv, cal.tau_k, cal.tau_v, 200, 32) for rv in (None, eye)]
    seqs = [[], []]
    for r, t in enumerate(lens0):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        for c in (0, 1):
            s = caches[c].new_seq()
            caches[c].append(s, kb, folded(vb))
            seqs[c].append(s)
    planners = [K.DecodeStepPlanner(caches[c].pool, seqs[c]) for c in (0, 1)]
    max_i2 = (max(lens0) + n_steps + 15) // 16
    max_bf = -(-sink // 16) + recent // 16 + 1
    ws = [torch.empty(K.oscar_decode_workspace_bytes(sh, B, 3, 1), dtype=torch.uint8, device="cuda") for _ in (0, 1)]
    outs = [torch.empty((B, hq, 128), dtype=torch.float32, device="cuda") for _ in (0, 1)]
    for st in range(n_steps):
        kn = np.stack([synth.kv_request_bf16(w, r, lens0[r] + st, lens0[r] + st + 1)[0][0] for r in range(B)])
        vn = np.stack([folded(synth.kv_request_bf16(w, r, lens0[r] + st, lens0[r] + st + 1)[1])[0]
                       for r in range(B)])
        q = to_dev_bits(np.stack([synth.q_decode_bf16(w, r, st + 1) for r in range(B)]))
        kd, vd = to_dev_bits(kn), to_dev_bits(vn)
        for c in (0, 1):
            planners[c].step()
            d = to_dev_i32(planners[c].buf)
            i2, bf, ctx = caches[c].tables(seqs[c], max_i2, max_bf)
            K.oscar_decode_step(sh, caches[c].layer, caches[c].cache, kd, vd, d[:4], q, to_dev_i32(i2),
                                to_dev_i32(bf), to_dev_i32(ctx), outs[c], ws[c], 3, 1)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1]), f"step {st}: r_v NULL and R_V = I differ"
    assert torch.equal(caches[0].int2, caches[1].int2) and torch.equal(caches[0].bf16, caches[1].bf16)
    out = outs[0].cpu().numpy()
    qf = np.stack([synth.q_decode_bf16(w, r, n_steps) for r in range(B)])
    for r in range(B):
        t = lens0[r] + n_steps
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        st_f = O.store_request(kb, folded(vb), cal_i, 32, sink, recent)
        _check_pages(caches[0], seqs[0][r], st_f, w, f"f4 folded len={t}")
        _check_close(out[r], O.decode_attention(qf[r], st_f, cal_i, 32), f"f4 folded decode len={t}")
        # rotated back, as accurate as the unfolded cache against exact attention
        back = np.stack([out[r][h].astype(np.float64) @ r_v64[h // (hq // hkv)].T for h in range(hq)])
        st_u = O.store_request(kb, vb, cal, 32, sink, recent)
        ex = O.attend(O.bf16_to_f64(qf[r]), O.bf16_to_f64(kb), O.bf16_to_f64(vb))
        e_f = np.linalg.norm(back - ex) / np.linalg.norm(ex)
        e_u = np.linalg.norm(O.decode_attention(qf[r], st_u, cal, 32) - ex) / np.linalg.norm(ex)
        _flush(f"f4 len={t}: error vs exact attention folded={e_f:.4f} unfolded={e_u:.4f}")
        # the folded projection's output carries its own bf16 rounding (2^-9 relative): the
        # only extra error, seen alone when every position is bf16
        assert e_f <= 1.05 * e_u + 2.0 ** -8, (t, e_f, e_u)


def _bits(vals):
    """float values exactly representable in bf16 -> bf16 bit patterns"""
    return synth.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _check_written_rows(dc, sh, kb, vb, r_k, r_v, tau_k, tau_v, group, scale_bits, label):
    pool = dc.int2.cpu().numpy().reshape(dc.int2.numel() // (sh.n_kv_heads * dc.int2_block), sh.n_kv_heads, -1)
    bits = np.uint16 if scale_bits == 16 else np.uint8
    n = kb.shape[0]
    for h in range(sh.n_kv_heads):
        ck, sk, zk, _ = O.quantize(O.bf16_to_f64(kb[:, h]), r_k[h], tau_k, group, scale_bits)
        cv, sv, zv, _ = O.quantize(O.bf16_to_f64(vb[:, h]), r_v[h], tau_v, group, scale_bits)
        bad = 0
        for i in range(n):
            page, s = divmod(i, 16)
            blk = O.unpack_int2_block(pool[page, h], 128, group, scale_bits)
            ok = (np.array_equal(blk[0][s], ck[i]) and np.array_equal(blk[3][s], cv[i])
                  and np.array_equal(blk[1][s].view(bits), sk[i].view(bits))
                  and np.array_equal(blk[2][s].view(bits), zk[i].view(bits))
                  and np.array_equal(blk[4][s].view(bits), sv[i].view(bits))
                  and np.array_equal(blk[5][s].view(bits), zv[i].view(bits)))
            if not ok:
                bad += 1
                if bad < 4:
                    _flush(f"{label}: head {h} token {i} differs")
        assert bad == 0, (label, h, bad)


@pytest.mark.parametrize("scale_bits", [16, 8])
@pytest.mark.parametrize("prepare", [True, False], ids=["prepared-digits", "derived-digits"])
def test_quant_write_certification_edges(scale_bits, prepare):
    """The write kernel's certified decisions at their edges, with identity
    rotations (R_K = I, R_V folded) so that the rotated values are the bf16
    inputs themselves: codes whose t is exactly a half-integer (the exact path
    breaks the tie half-even), groups with s = 0, values clipped at +-tau,
    entries far below the token's maximum (rounded in the fixed point, covered
    by the bound), an all-zero token and a ragged tail; then a rotation with
    entries outside [-1.5, 1.5], which sends every tile to the exact path."""
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    w = synth.WORKLOADS["qwen3_8b_32k"]
    sh = K.make_shape(n_q_heads=4, n_kv_heads=1, group=32, sink=0, recent=0, scale_bits=scale_bits)
    n = 19 * 16 + 5
    kb, vb = synth.kv_request_bf16(w, 11, 0, n)
    kb, vb = np.ascontiguousarray(kb[:, :1]), np.ascontiguousarray(vb[:, :1])
    rng = np.random.default_rng(5)
    ties = np.array([0.0, 3.0, 0.5, 1.5, 2.5] * 26)[:128]       # z = 0, s = 1, t on .5 boundaries
    for x in (kb, vb):
        x[0] = 0                                                  # all-zero token
        x[1, 0] = _bits(ties)
        x[2, 0] = _bits(ties * 0.25 - 0.375)                      # shifted and scaled ties
        tiny = np.full(128, 2.0 ** -30)
        tiny[::7] = 2.0 ** -40
        tiny[3], tiny[64] = 1.0, -0.75
        x[3, 0] = _bits(tiny)                                     # entries 2^-30, 2^-40 below max 1
        x[4, 0] = _bits(np.full(128, 0.75))                       # s = 0 in every group
        x[5, 0] = _bits(np.where(np.arange(128) % 3 == 0, 10.0, -0.3))  # clipped at tau
        for t in range(6, 40):                                    # random small integers and halves: many ties
            x[t, 0] = _bits(rng.integers(-6, 7, 128) * 0.5)
    eye = np.eye(128, dtype=np.float32)[None]
    for label, r_k, tau in (("identity", eye, 4.0), ("R outside [-1.5, 1.5]", 2.0 * eye, 8.0)):
        _flush(f"case certification edges: {label}, scale_bits {scale_bits}")
        dc = DeviceCache(sh, r_k, None, tau, tau, (n + 15) // 16, 1, prepare=prepare)
        K.oscar_quant_write(sh, dc.layer, dc.cache, to_dev_bits(kb), to_dev_bits(vb),
                            to_dev_i32(np.arange(n, dtype=np.int32)))
        torch.cuda.synchronize()
        _check_written_rows(dc, sh, kb, vb, r_k.astype(np.float64), eye.astype(np.float64), tau, tau, 32,
                            scale_bits, label)


@pytest.mark.parametrize("group,scale_bits", [(32, 16), (64, 8)])
def test_prepared_digits_match_derived(group, scale_bits):
    """R's digits prepared once per layer (oscar_layer_prepare) against the
    ones every write work group derives: identical INT2 bytes for the same
    writes (a 16384-token chunk and a 4096-token one, x40 outliers, the
    calibrated rotations, and R_V folded), and the prepared buffer itself
    identical across two preparations."""
    from kv_cache_int2_amd.torch_cache import to_dev_bits, to_dev_i32
    w = synth.Workload("prep", 90 + group, 96, 8, 128, 1, 0, group=group, sink=4, recent=128,
                       outlier_scale=(40.0, 40.0), calib_tokens=1024)
    cal = _calibrate(w)
    sh = K.make_shape(n_q_heads=96, n_kv_heads=8, group=group, sink=4, recent=128, scale_bits=scale_bits)
    n = 16384 + 4096
    kb, vb = synth.kv_request_bf16(w, 3, 0, n)
    for r_v in (cal.r_v, None):
        label = "R_V folded" if r_v is None else "calibrated"
        _flush(f"case prepared digits G={group} scale_bits={scale_bits} {label}")
        caches = [DeviceCache(sh, cal.r_k, r_v, cal.tau_k, cal.tau_v, n // 16 + 1, 1, prepare=pr)
                  for pr in (True, False)]
        again = torch.empty_like(caches[0].r_prep)
        K.oscar_layer_prepare(sh, caches[0].layer, again)
        for dc in caches:
            for a, b in ((0, 16384), (16384, n)):   # a 16384-token call and a 4096-token one
                K.oscar_quant_write(sh, dc.layer, dc.cache, to_dev_bits(kb[a:b]), to_dev_bits(vb[a:b]),
                                    to_dev_i32(np.arange(a, b, dtype=np.int32)))
        torch.cuda.synchronize()
        assert torch.equal(caches[0].r_prep, again), label
        assert torch.equal(caches[0].int2, caches[1].int2), label

