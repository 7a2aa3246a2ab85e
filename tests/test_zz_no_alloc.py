"""The allocation-free decode entry point, oscar_decode_attn_noalloc (its
split-K workspace is a device array inside the library), against
oscar_decode_attn with a caller workspace: bit-identical outputs on two calls
in a row, the second with a smaller batch and other split counts (the array
then holds the first call's bytes), and both within tolerance of the fp64
oracle.  A call that needs more workspace than the array holds is refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import kv_cache_int2_amd as K
import oracle as O
import synth
from kv_cache_int2_amd.torch_cache import DeviceCache, to_dev_bits, to_dev_i32

pytestmark = pytest.mark.gpu

MAX_ABS, REL_L2 = 2e-3, 1e-3


def _flush(msg):
    print(msg, flush=True)


def test_noalloc_decode_matches_the_workspace_entry_point():
    hq, hkv, group, sink, recent = 32, 8, 32, 4, 32
    w = synth.Workload("noalloc", 91, hq, hkv, 128, 1, 0, group=group, sink=sink, recent=recent,
                       outlier_scale=(20.0, 20.0), calib_tokens=512)
    _flush("case noalloc decode: 6 then 3 requests, 32q/8kv, G=32")
    q, k, v = synth.calib_layer(w)
    cal = O.calibrate_layer(q, k, v)
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=group, sink=sink, recent=recent)
    lens = [3001, 1, 700, 2049, 37, 1500]
    dc = DeviceCache(sh, cal.r_k, cal.r_v, cal.tau_k, cal.tau_v, sum(t // 16 + 2 for t in lens), 64)
    seqs, stores = [], {}
    for r, t in enumerate(lens):
        kb, vb = synth.kv_request_bf16(w, r, 0, t)
        seq = dc.new_seq()
        dc.append(seq, kb, vb)
        seqs.append(seq)
        if r in (0, 2, 3):
            stores[r] = O.store_request(kb, vb, cal, group, sink, recent)
    qs = np.stack([synth.q_decode_bf16(w, r) for r in range(len(lens))])
    # the second call is smaller (3 requests) and uses other split counts
    for call, (idx, si, sb) in enumerate((([0, 1, 2, 3, 4, 5], 0, 4), ([3, 1, 2], 3, 2))):
        _flush(f"case noalloc call {call}: requests {idx}, splits {si}/{sb}")
        i2, bf, ctx = dc.tables([seqs[i] for i in idx])
        i2d, bfd, ctxd = to_dev_i32(i2), to_dev_i32(bf), to_dev_i32(ctx)
        qd = to_dev_bits(qs[idx])
        si_r = si or K.oscar_decode_auto_splits(sh, len(idx), i2.shape[1])
        need = K.oscar_decode_workspace_bytes(sh, len(idx), si_r, sb)
        assert need <= K.oscar_decode_noalloc_max_workspace_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref = torch.empty((len(idx), hq, 128), dtype=torch.float32, device="cuda")
        out = torch.full_like(ref, float("nan"))
        K.oscar_decode_attn(sh, dc.layer, dc.cache, qd, i2d, bfd, ctxd, ref, ws, si_r, sb)
        K.oscar_decode_attn_noalloc(sh, dc.layer, dc.cache, qd, i2d, bfd, ctxd, out, si, sb)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {call}: outputs differ from oscar_decode_attn"
        out_np = out.cpu().numpy()
        for j, r in enumerate(idx):
            if r in stores:
                exp = O.decode_attention(qs[r], stores[r], cal, group)
                err = float(np.abs(out_np[j] - exp).max())
                rel = float(np.linalg.norm(out_np[j] - exp) / np.linalg.norm(exp))
                _flush(f"noalloc call {call} request {r} len={lens[r]}: max_abs={err:.3e} rel_l2={rel:.3e}")
                assert err <= MAX_ABS and rel <= REL_L2, (call, r, err, rel)


def test_noalloc_decode_refuses_more_than_its_workspace():
    """A batch whose split-K workspace exceeds the library's array is refused
    with OSCAR_EINVAL and a message naming the limit; nothing is enqueued (the
    output keeps its NaN fill)."""
    hq, hkv = 32, 8
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=32, sink=4, recent=32)
    cap = K.oscar_decode_noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    batch, si, sb = 2048, 64, 4
    assert K.oscar_decode_workspace_bytes(sh, batch, si, sb) > cap
    _flush(f"case noalloc refusal: batch {batch}, splits {si}/{sb}")
    rk = torch.zeros((hkv, 128, 128), dtype=torch.float32, device="cuda")
    lay = K.make_layer(rk, rk, 1.0, 1.0)
    blk_i2, blk_bf = K.oscar_int2_block_bytes(sh), K.oscar_bf16_block_bytes(sh)
    i2pool = torch.zeros(4 * hkv * blk_i2, dtype=torch.uint8, device="cuda")
    bfpool = torch.zeros(4 * hkv * blk_bf, dtype=torch.uint8, device="cuda")
    cache = K.make_cache(i2pool, 4, bfpool, 4)
    q = torch.zeros((batch, hq, 128), dtype=torch.int16, device="cuda")
    tab = torch.zeros((batch, 1), dtype=torch.int32, device="cuda")
    ctx = torch.zeros(batch, dtype=torch.int32, device="cuda")
    out = torch.full((batch, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(K.OscarError) as ei:
        K.oscar_decode_attn_noalloc(sh, lay, cache, q, tab, tab, ctx, out, si, sb)
    assert ei.value.code == K.OSCAR_EINVAL
    assert "allocation-free" in str(ei.value)
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
