"""Benchmark of the OSCAR INT2 KV-cache hot path on one MI355X.

One step = one decode step for the whole batch: host region planning
(oscar_plan_decode_step), then oscar_decode_step: re-quantisation of the
tokens leaving the recent window and bf16 append of every request's new token
(fused into the prologue kernel), and mixed-precision paged decode attention
(prologue, INT2 kernel, split-K combine running the bf16 region first).  --unfused runs
the same step with the writes as separate calls.  The cache is resident in
HBM before the timed region; the inputs of the steps are generated and
uploaded beforehand (128 distinct sets, used in turn).

Prints one JSON line.  value = KV tokens attended per second (summed context
lengths of all requests and steps / wall time of the timed steps).
"""
from __future__ import annotations

import argparse
import ctypes as C
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA
WRITE_DIGIT_PAIRS = 16         # int8 digit-pair products per rotation in the write kernel
PROFILE_PMC = os.path.join(ROOT, "profiles", "decode_int2_long_28x100k_pmc.json")
KERNEL_SRC = os.path.join(ROOT, "kv_cache_int2_amd", "csrc", "decode_attn.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed decode steps before the timed ones (after the settle phase)")
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="untimed clock-settle phase first: read-only decode launches on the filled cache for "
                         "this long (wall ms), running straight into the warm-up and timed steps, so that the "
                         "GPU's power management has left its post-idle ramp before any timed step")
    ap.add_argument("--workload", default="long_28x100k")
    ap.add_argument("--group", type=int, default=0, help="override the workload's INT2 group size")
    ap.add_argument("--layout", choices=["workload", "pages"], default="workload",
                    help="pages: the pages' default layout (sink 64, recent 256, G = 64, FP8 scale and zero)")
    ap.add_argument("--splits", type=int, default=0, help="INT2 splits per (request, KV head); 0 = auto")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch (requests)")
    ap.add_argument("--context", type=int, default=0, help="override the workload's context length (tokens)")
    ap.add_argument("--decode-form", choices=["auto", "standard", "small"], default="auto",
                    help="decode launch form (oscar_decode_set_small_grid): auto, standard (one combine work "
                         "group per (request, KV head)), small (bf16 splits inside the INT2 kernel's grid, one "
                         "combine work group per query head, where one wavefront holds an item's tiles)")
    ap.add_argument("--mode", choices=["decode", "prefill"], default="decode",
                    help="prefill: time chunked-prefill attention (oscar_prefill_attn) of --chunk queries per "
                         "request over the filled cache instead of decode steps")
    ap.add_argument("--chunk", type=int, default=128, help="queries per request in --mode prefill")
    ap.add_argument("--unfused", action="store_true",
                    help="separate write calls and in-order kernels instead of the fused decode step")
    ap.add_argument("--interleave", action="store_true",
                    help="each step also runs the workload's chunked-prefill writes (stress 16x128k: 16 chunks of "
                         "4096 tokens, bf16 in, quant_write) into a separate page pool, on the same stream")
    ap.add_argument("--interleave-batched", action="store_true",
                    help="with --interleave: the step's chunks in one quant_write call (all their tokens and "
                         "slots), as a serving step writes its whole prefill batch, instead of one call per chunk")
    ap.add_argument("--cold-flush-mb", type=int, default=0,
                    help="before every step, overwrite a buffer of this many MB (above the 256 MB MALL: the step "
                         "reads its cache cold); the step's GPU time is then taken from events around it")
    ap.add_argument("--no-baseline", action="store_true", help="skip the bf16 same-kernel baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


def int2_tokens(t, sink, recent):
    """INT2 history tokens of a request of length t: positions [sink, t - recent)."""
    return max(0, int(t) - sink - recent)


def algorithmic_bytes(ctx, hkv, hq, group, sink, recent, mb=4):
    """Bytes the method must move for one decode of the batch: INT2 codes +
    scale/zero of history tokens, bf16 K/V of sink/recent tokens, the bf16
    query and the fp32 output."""
    per_int2 = 2 * (128 // 4 + (128 // group) * mb)         # K and V, per token and KV head
    per_bf16 = 2 * 128 * 2
    tot = 0
    for t in ctx:
        n_i2 = int2_tokens(t, sink, recent)
        tot += (n_i2 * per_int2 + (int(t) - n_i2) * per_bf16) * hkv
    return tot + len(ctx) * hq * 128 * (2 + 4)


def int2_kernel_bytes(ctx, hkv, group, sink, recent, mb=4):
    """Algorithmic bytes of one launch of the INT2 kernel: 2 x (32 B of codes +
    (128/G) x mb B of scale/zero, mb = 4 for fp16, 2 for FP8) per INT2 token
    and KV head (96 B at G=32 fp16, 80 B at G=64 fp16, 72 B at G=64 FP8).  The
    bf16 tokens belong to the bf16 region's work."""
    per_int2 = 2 * (128 // 4 + (128 // group) * mb)
    return sum(int2_tokens(t, sink, recent) for t in ctx) * hkv * per_int2


def settle_clocks(settle_ms, launch):
    """Untimed clock-settle phase: call launch() (a read-only decode of the
    filled cache) in batches of 25 until settle_ms of wall time have passed.
    After an idle spell the GPU's power management needs ~50 launches of
    sustained load before the decode kernel runs at its steady speed again,
    so the steps must follow this phase with no host pause: the caller reads
    the recorded per-launch durations only after its timed steps.  Returns
    (launches, wall ms)."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(25):
            launch()
        n += 25
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def settle_summary(each_us, wall_ms):
    marks = [m for m in (1, 10, 25, 50, 100, 200, 400, 800, 1600, 3200, 6400) if m <= each_us.size]
    curve = {str(m): round(float(each_us[max(0, m - 25):m].mean()), 1) for m in marks}
    log(f"settle: {each_us.size} read-only decode launches in {wall_ms:.0f} ms; decode_int2 us by launch index "
        f"(mean of the 25 before): {curve}" + (f"; last 100 mean {each_us[-100:].mean():.1f}" if each_us.size else ""))
    return {"ms": round(wall_ms, 1), "launches": int(each_us.size), "kind": "read-only decode of the filled cache",
            "kernel_us_first": round(float(each_us[0]), 2) if each_us.size else None,
            "kernel_us_last100": round(float(each_us[-100:].mean()), 2) if each_us.size else None,
            "kernel_us_by_launch": curve}


def run_prefill(args, w, sh, group, scale_bits, mb, cal):
    """Chunked prefill: every request holds T - C tokens, its C-token chunk is
    written, then the chunk's queries attend over the mixed cache; the
    attention launches (oscar_prefill_attn) are timed, the cache unchanged."""
    import torch
    import kv_cache_int2_amd as K
    import synth
    from kv_cache_int2_amd.torch_cache import DeviceCache, to_dev_bits, to_dev_i32
    B, hq, hkv, T, C = w.batch, w.n_q_heads, w.n_kv_heads, w.context, args.chunk
    r_k, r_v, tau_k, tau_v = cal
    ppr = (T + 15) // 16 + 2
    dc = DeviceCache(sh, r_k, r_v, tau_k, tau_v, B * ppr + 8, B * (w.sink // 16 + 2 + w.recent // 16) + 8)
    seqs = []
    t = time.time()
    for r in range(B):
        kb, vb = synth.kv_request_bf16(w, r, 0, T)
        s = dc.new_seq()
        for c0 in range(0, T - C, 16384):
            c1 = min(T - C, c0 + 16384)
            dc.append(s, kb[c0:c1], vb[c0:c1])
        dc.append(s, kb[T - C:], vb[T - C:])        # the chunk
        seqs.append(s)
    torch.cuda.synchronize()
    log(f"cache filled in {time.time() - t:.1f}s; chunk of {C} per request written")
    i2, bf, ctx = dc.tables(seqs)
    q = to_dev_bits(np.stack([np.stack([synth.q_decode_bf16(w, r, c) for c in range(C)]) for r in range(B)]))
    ws = torch.empty(K.oscar_prefill_workspace_bytes(sh, B, C), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, C, hq, 128), dtype=torch.float32, device="cuda")
    i2d, bfd, ctxd = to_dev_i32(i2), to_dev_i32(bf), to_dev_i32(ctx)
    for _ in range(args.warmup):
        K.oscar_prefill_attn(sh, dc.layer, dc.cache, q, i2d, bfd, ctxd, out, ws)
    torch.cuda.synchronize()
    K.oscar_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        K.oscar_prefill_attn(sh, dc.layer, dc.cache, q, i2d, bfd, ctxd, out, ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    K.oscar_profile_enable(False)
    int2_ms, launches = K.oscar_profile_read()
    assert torch.isfinite(out).all(), "non-finite prefill output"
    ctx_np = ctx.astype(np.int64)
    attended = int(sum(int(c) - C + i + 1 for c in ctx_np for i in range(C)))
    per_call = (t1 - t0) / args.steps
    int2_us = int2_ms / max(launches, 1) * 1e3
    int2_bytes = int2_kernel_bytes(ctx_np, hkv, group, w.sink, w.recent, mb)
    log(f"prefill: {per_call * 1e3:.3f} ms per call, {launches // max(args.steps, 1)} INT2 passes of "
        f"{int2_us:.1f} us each")
    res = {
        "metric": "chunked-prefill attention over the mixed cache: KV tokens attended/s",
        "value": attended / per_call, "unit": "KV tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": per_call * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8+f16 mfma, f32 acc", "data": "synthetic (seeded generator)",
        "config": {"workload": w.name, "batch": B, "context": T, "chunk": C, "n_q_heads": hq, "n_kv_heads": hkv,
                   "group": group, "sink": w.sink, "recent": w.recent, "scale_bits": scale_bits},
        "int2_pass": {"kernel": "decode_int2", "passes_per_call": launches // max(args.steps, 1),
                      "us_per_pass": round(int2_us, 2), "int2_bytes_per_pass": int(int2_bytes),
                      "gbs_per_pass": round(int2_bytes / (int2_us * 1e-6) / 1e9, 1)},
        # one pass reads the INT2 history once for 16 queries' rows: its bytes
        # against HBM; the pass is bound by its VALU and MFMA issue, which the
        # SQ counters of the profile show
        "roofline": {"bound": "hbm", "achieved": round(int2_bytes / (int2_us * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(int2_bytes / (int2_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_int2", "kernel_us": round(int2_us, 2),
                     "algorithmic_bytes_per_launch": int(int2_bytes)},
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: there is no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_cache_int2_amd as K
    import synth
    from kv_cache_int2_amd.torch_cache import BaselineCache, DeviceCache, to_dev_bits, to_dev_i32

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    scale_bits = 16
    if args.layout == "pages":
        w = dataclasses.replace(w, sink=64, recent=256, group=64)
        scale_bits = 8
    if args.batch:
        w = dataclasses.replace(w, batch=args.batch)
    if args.context:
        w = dataclasses.replace(w, context=args.context)
    K.oscar_decode_set_small_grid({"auto": 0, "standard": 1, "small": 2}[args.decode_form])
    group = args.group or w.group
    mb = 4 if scale_bits == 16 else 2
    B, hq, hkv = w.batch, w.n_q_heads, w.n_kv_heads
    n_steps = args.warmup + args.steps
    T_final = w.context
    T0 = T_final - n_steps                      # the last timed step attends T_final tokens
    sh = K.make_shape(n_q_heads=hq, n_kv_heads=hkv, group=group, sink=w.sink, recent=w.recent,
                      scale_bits=scale_bits)
    log(f"workload {w.name}: B={B} T={T_final} Hq={hq} Hkv={hkv} G={group} sink={w.sink} recent={w.recent} "
        f"scale_bits={scale_bits}")

    # ---- calibration (offline, host C++) ----
    t = time.time()
    qc, kc, vc = synth.calib_layer(w)
    r_k, r_v, _, _, tau_k, tau_v = K.oscar_calibrate_host(sh, qc, kc, vc)
    log(f"calibration {time.time() - t:.1f}s tau_k={tau_k:.3f} tau_v={tau_v:.3f}")
    if args.mode == "prefill":
        run_prefill(args, w, sh, group, scale_bits, mb, (r_k, r_v, tau_k, tau_v))
        return

    pages_per_req = (T_final + 15) // 16 + 2
    dc = DeviceCache(sh, r_k, r_v, tau_k, tau_v, B * pages_per_req + 8, B * (w.sink // 16 + 2 + w.recent // 16) + 8)
    bc = None
    if not args.no_baseline:
        bc = BaselineCache(sh, B * pages_per_req + 8, T_final + 16)

    # ---- fill the cache (prefill through the write path, timed per quant_write launch) ----
    seqs, bseqs = [], []
    qw_ms, qw_tokens = [], 0
    chunk = 16384
    t = time.time()
    parent = None
    if w.shared_prefix:
        kb, vb = synth.kv_request_bf16(w, 0, 0, w.shared_prefix)
        parent = dc.new_seq()
        dc.append(parent, kb, vb)
        pbk, pbv = kb, vb
    for r in range(B):
        start = 0
        if parent is not None:
            s = dc.fork(parent)
            start = w.shared_prefix
        else:
            s = dc.new_seq()
        kb_all, vb_all = synth.kv_request_bf16(w, r, start, T0)
        if bc is not None:
            bs = bc.new_seq()
            if parent is not None:
                bc.append(bs, pbk, pbv)
        for c0 in range(0, T0 - start, chunk):
            kb, vb = kb_all[c0:c0 + chunk], vb_all[c0:c0 + chunk]
            i2, bf, a_s, a_d = K.oscar_seq_plan_append(dc.pool, s, kb.shape[0])
            kd, vd = to_dev_bits(kb), to_dev_bits(vb)
            if len(a_s):
                K.oscar_requant_from_bf16(sh, dc.layer, dc.cache, to_dev_i32(a_s), to_dev_i32(a_d))
            if np.any(i2 >= 0):
                i2d = to_dev_i32(i2)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                K.oscar_quant_write(sh, dc.layer, dc.cache, kd, vd, i2d)
                e1.record()
                qw_ms.append((e0, e1))
                qw_tokens += int(np.count_nonzero(i2 >= 0))
            if np.any(bf >= 0):
                K.oscar_bf16_write(sh, dc.cache, kd, vd, to_dev_i32(bf))
            if bc is not None:
                bc.append(bs, kb, vb)
        seqs.append(s)
        if bc is not None:
            bseqs.append(bs)
        del kb_all, vb_all
        if r % 7 == 0:
            log(f"filled request {r + 1}/{B} ({time.time() - t:.1f}s)")
    torch.cuda.synchronize()
    qw_time = sum(a.elapsed_time(b) for a, b in qw_ms) / 1e3
    log(f"cache filled in {time.time() - t:.1f}s; quant_write {qw_tokens} tokens in {qw_time * 1e3:.1f} ms")

    # ---- step inputs, resident before timing (n_in distinct sets, used in turn) ----
    n_in = min(n_steps, 128)
    new_k = np.empty((n_in, B, hkv, 128), np.uint16)
    new_v = np.empty_like(new_k)
    qs = np.empty((n_in, B, hq, 128), np.uint16)
    for r in range(B):
        kb, vb = synth.kv_request_bf16(w, r, T0, T0 + n_in, threads=1)
        new_k[:, r], new_v[:, r] = kb, vb
        for st in range(n_in):
            qs[st, r] = synth.q_decode_bf16(w, r, st + 1)
    new_k_d, new_v_d, q_d = to_dev_bits(new_k), to_dev_bits(new_v), to_dev_bits(qs)
    planner = K.DecodeStepPlanner(dc.pool, seqs)
    host_small = torch.zeros((n_steps, 5, B), dtype=torch.int32).pin_memory()
    dev_small = torch.zeros((n_steps, 5, B), dtype=torch.int32, device="cuda")
    max_i2 = (T_final + 15) // 16
    max_bf = w.sink // 16 + 1 + w.recent // 16
    si = args.splits or K.oscar_decode_auto_splits(sh, B, max_i2)
    sb_step = 4                                 # bf16 splits, run inside the combine kernel
    ws = torch.empty(K.oscar_decode_workspace_bytes(sh, B, si, sb_step), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    i2_bt, bf_bt, ctx = dc.tables(seqs, max_i2, max_bf)
    tables = [to_dev_i32(i2_bt), to_dev_i32(bf_bt)]
    ctx_hist = []
    # block-table refreshes (a new page every 16 steps) go up from a ring of
    # pinned buffers without blocking the host, as a serving loop sends them: a
    # copy from pageable memory would wait for every queued kernel and leave
    # the GPU idle while the host queues the next step.  A slot is rewritten
    # only after its previous copy has completed (its event).
    n_tab = 4
    tab_host = [(torch.empty(i2_bt.shape, dtype=torch.int32).pin_memory(),
                 torch.empty(bf_bt.shape, dtype=torch.int32).pin_memory()) for _ in range(n_tab)]
    tab_dev = [(torch.empty(i2_bt.shape, dtype=torch.int32, device="cuda"),
                torch.empty(bf_bt.shape, dtype=torch.int32, device="cuda")) for _ in range(n_tab)]
    tab_ev = [None] * n_tab
    tab_n = [0]

    # chunked-prefill writes of other requests, interleaved with each step:
    # inputs resident in HBM, destinations a page pool of their own
    iw = None
    if args.interleave:
        if not w.write_chunks:
            raise SystemExit(f"workload {w.name} defines no interleaved write chunks")
        nc, ct = w.write_chunks, w.write_chunk
        n_w = nc * ct
        dcw = DeviceCache(sh, r_k, r_v, tau_k, tau_v, n_w // 16 + 1, 1)
        kw = np.empty((n_w, hkv, 128), np.uint16)
        vw = np.empty_like(kw)
        for c in range(nc):
            kw[c * ct:(c + 1) * ct], vw[c * ct:(c + 1) * ct] = synth.kv_request_bf16(w, 100_000 + c, 0, ct)
        iw = (nc, ct, dcw, to_dev_bits(kw), to_dev_bits(vw), to_dev_i32(np.arange(n_w, dtype=np.int32)))
        del kw, vw
        log(f"interleaved writes: {nc} chunks x {ct} tokens per step")
    flush = torch.empty(args.cold_flush_mb << 20, dtype=torch.uint8, device="cuda") if args.cold_flush_mb else None
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    # events around each step cost the queue a few microseconds per step: the
    # timed steps carry them only where their time is the measure (cold-cache
    # steps, whose flush the wall time holds, and the interleaved-write runs);
    # otherwise the step's GPU time is read from the warm-up steps
    timed_step_ev = flush is not None or iw is not None
    step_ev_range = range(args.warmup, n_steps) if timed_step_ev or args.warmup == 0 else range(args.warmup)
    write_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]

    # up to 64 requests the step's slot table and lengths travel in the prologue's
    # launch arguments (oscar_decode_step_host_tables): no copy per step
    host_tables = not args.unfused and B <= 64

    # the host-table step's pointer arguments, marshalled once: the binding's
    # per-call conversions (about 4 us) would set the pace of a one-request step
    step_fn = K.lib().oscar_decode_step_host_tables
    step_args = {"slots": planner.buf.ctypes.data, "ctx": planner.buf.ctypes.data + 4 * planner.buf.shape[1] * 4,
                 "head": (C.byref(sh), C.byref(dc.layer), C.byref(dc.cache)),
                 "io": [(new_k_d[i].data_ptr(), new_v_d[i].data_ptr(), q_d[i].data_ptr()) for i in range(n_in)],
                 "tail": (out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                          torch.cuda.current_stream().cuda_stream),
                 "tables": None}

    def step(st):
        n_age, changed = planner.step()
        if not host_tables:
            host_small[st].copy_(torch.from_numpy(planner.buf))
            dev_small[st].copy_(host_small[st], non_blocking=True)
        if changed:
            i2_bt, bf_bt, _ = dc.tables(seqs, max_i2, max_bf)
            k = tab_n[0] % n_tab
            tab_n[0] += 1
            if tab_ev[k] is not None:
                tab_ev[k].synchronize()
            for hb, db, a in zip(tab_host[k], tab_dev[k], (i2_bt, bf_bt)):
                hb.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)))
                db.copy_(hb, non_blocking=True)
            tab_ev[k] = torch.cuda.Event()
            tab_ev[k].record()
            tables[0], tables[1] = tab_dev[k]
            step_args["tables"] = None
        d = dev_small[st]
        si_ = st % n_in
        if flush is not None:
            flush.fill_(st & 0xFF)
        ev = st in step_ev_range
        if ev:
            step_ev[st][0].record()
        if args.unfused:
            if n_age:
                K.oscar_requant_from_bf16(sh, dc.layer, dc.cache, d[2], d[3], n=B)
            if np.any(planner.buf[0] >= 0):
                K.oscar_quant_write(sh, dc.layer, dc.cache, new_k_d[si_], new_v_d[si_], d[0], n=B)
            K.oscar_bf16_write(sh, dc.cache, new_k_d[si_], new_v_d[si_], d[1], n=B)
            K.oscar_decode_attn(sh, dc.layer, dc.cache, q_d[si_], tables[0], tables[1], d[4], out, ws, si, sb_step)
        elif host_tables:
            # oscar_decode_step_host_tables(shape, layer, cache, k_new, v_new, step_slots, q, batch, int2_bt,
            # max_int2_pages, bf16_bt, max_bf16_pages, ctx_lens, splits_int2, splits_bf16, out, workspace,
            # workspace_bytes, stream), as the binding's wrapper passes them
            if step_args["tables"] is None:
                step_args["tables"] = (tables[0].data_ptr(), tables[0].shape[1], tables[1].data_ptr(),
                                       tables[1].shape[1])
            kp, vp, qp = step_args["io"][si_]
            i2p, i2n, bfp, bfn = step_args["tables"]
            K._check(step_fn(*step_args["head"], kp, vp, step_args["slots"], qp, B, i2p, i2n, bfp, bfn,
                             step_args["ctx"], si, sb_step, *step_args["tail"]))
        else:
            K.oscar_decode_step(sh, dc.layer, dc.cache, new_k_d[si_], new_v_d[si_], d[:4], q_d[si_], tables[0],
                                tables[1], d[4], out, ws, si, sb_step)
        if ev:
            step_ev[st][1].record()
        if iw is not None:
            nc, ct, dcw, kw_d, vw_d, slots_w = iw
            write_ev[st][0].record()
            if args.interleave_batched:
                K.oscar_quant_write(sh, dcw.layer, dcw.cache, kw_d, vw_d, slots_w)
            else:
                for c in range(nc):
                    K.oscar_quant_write(sh, dcw.layer, dcw.cache, kw_d[c * ct:(c + 1) * ct],
                                        vw_d[c * ct:(c + 1) * ct], slots_w[c * ct:(c + 1) * ct])
            write_ev[st][1].record()
        ctx_hist.append(planner.buf[4].astype(np.int64).copy())

    # ---- clock settle: read-only decode of the filled cache, untimed, for a fixed wall time ----
    # Clock settle, warm-up and timed steps run back to back with the decode
    # kernel's events recorded throughout and read only at the end: a host
    # pause between the phases would idle the GPU and restart its clock ramp.
    ctx_d0 = to_dev_i32(ctx)
    K.oscar_profile_enable(True)
    n_settle, settle_wall = settle_clocks(args.settle_ms, lambda: K.oscar_decode_attn(
        sh, dc.layer, dc.cache, q_d[0], tables[0], tables[1], ctx_d0, out, ws, si, sb_step))
    for st in range(args.warmup):
        step(st)
    torch.cuda.synchronize()
    ctx_hist.clear()
    t0 = time.perf_counter()
    for st in range(args.warmup, n_steps):
        step(st)
    t_issued = time.perf_counter()  # the host has queued every step; near t1 means the host sets the pace
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    K.oscar_profile_enable(False)
    _, n_ev, all_ms = K.oscar_profile_read_each(n_settle + n_steps + 16)
    assert n_ev == n_settle + n_steps, (n_ev, n_settle, n_steps)
    settle = settle_summary(all_ms[:n_settle] * 1e3, settle_wall)
    warm_ms = all_ms[n_settle:n_settle + args.warmup]
    each_ms = all_ms[n_settle + args.warmup:]
    launches = each_ms.size
    main_ms = float(each_ms.sum())
    if warm_ms.size:
        log("warm-up decode_int2 us: " + " ".join(f"{v * 1e3:.0f}" for v in warm_ms[:32]))
    step_gpu_us = float(np.mean([step_ev[i][0].elapsed_time(step_ev[i][1]) for i in step_ev_range])) * 1e3
    interleaved = None
    if iw is not None:
        nc, ct = iw[0], iw[1]
        n_w = nc * ct
        wr_us = float(np.mean([a.elapsed_time(b) for a, b in write_ev[args.warmup:]])) * 1e3
        wr_bytes = n_w * hkv * (2 * 128 * 2 + 2 * (32 + (128 // group) * mb))
        interleaved = {"chunks": nc, "chunk_tokens": ct, "calls_per_step": 1 if args.interleave_batched else nc,
                       "us_per_step": round(wr_us, 1),
                       "tokens_per_s": n_w / (wr_us * 1e-6), "bytes_per_step": wr_bytes,
                       "gbs": round(wr_bytes / (wr_us * 1e-6) / 1e9, 1),
                       "frac": round(wr_bytes / (wr_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"interleaved writes: {wr_us:.1f} us per step for {n_w} tokens ({interleaved['gbs']} GB/s); "
            f"decode step on the GPU {step_gpu_us:.1f} us")
    elapsed = t1 - t0
    tokens = int(sum(c.sum() for c in ctx_hist))
    value = tokens / elapsed
    value_basis = "wall time of the timed steps" + (" (each with its interleaved writes)" if iw is not None else "")
    if flush is not None:
        # the wall time holds the cache flushes: count the steps' own GPU time
        elapsed = step_gpu_us * 1e-6 * args.steps
        value = tokens / elapsed
        value_basis = "GPU time of the timed steps (events around each step; the flush before it excluded)"
    main_avg_ms = main_ms / max(launches, 1)
    alg_step = np.mean([algorithmic_bytes(c, hkv, hq, group, w.sink, w.recent, mb) for c in ctx_hist])
    alg = np.mean([int2_kernel_bytes(c, hkv, group, w.sink, w.recent, mb) for c in ctx_hist])
    achieved = alg / (main_avg_ms * 1e-3) / 1e9
    # shared-prefix batches: the prefix's complete INT2 pages ([sink, prefix - recent)) are one
    # physical copy read by every request; count them once for the HBM roofline
    alg_unique = alg
    if w.shared_prefix:
        shared_i2 = max(0, w.shared_prefix - w.recent - w.sink)
        alg_unique = alg - (B - 1) * shared_i2 * hkv * 2 * (32 + (128 // group) * mb)
        log(f"shared prefix: INT2 bytes per launch {alg:.0f} logical, {alg_unique:.0f} unique "
            f"({alg_unique / (main_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS:.1%} of peak on unique bytes)")
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms: {value / 1e9:.3f} G KV tok/s; "
        f"decode_int2 avg {main_avg_ms * 1e3:.1f} us -> {achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS:.1%} of peak)")
    log("decode_int2 us per timed step: " + " ".join(f"{v * 1e3:.0f}" for v in each_ms[:64]))

    # ---- parity sample on the timed cache: cheap invariant (finite output) ----
    assert torch.isfinite(out).all(), "non-finite decode output"

    # ---- HBM traffic from committed rocprofv3 counters (if they match this kernel source) ----
    traffic = None
    src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if os.path.exists(PROFILE_PMC):
        pm = json.load(open(PROFILE_PMC))
        if pm.get("kernel_source_sha256") == src_hash and pm.get("workload") == w.name:
            traffic = pm.get("hbm_bytes_per_launch")

    # ---- bf16 same-kernel baseline ----
    baseline = None
    if bc is not None:
        bq = q_d[(n_steps - 1) % n_in]
        btab = bc.tables(bseqs)
        bf_bt_d, bctx = to_dev_i32(btab[0]), to_dev_i32(btab[1])
        sb = K.oscar_decode_auto_splits(bc.shape, B, btab[0].shape[1])
        bws = torch.empty(K.oscar_decode_workspace_bytes(bc.shape, B, 1, sb), dtype=torch.uint8, device="cuda")
        bout = torch.empty_like(out)
        for _ in range(3):
            K.oscar_decode_attn_bf16_baseline(bc.shape, bc.cache, bq, bf_bt_d, bctx, bout, bws, sb)
        torch.cuda.synchronize()
        K.oscar_profile_enable(True)
        nb = max(5, args.steps // 2)
        tb0 = time.perf_counter()
        for _ in range(nb):
            K.oscar_decode_attn_bf16_baseline(bc.shape, bc.cache, bq, bf_bt_d, bctx, bout, bws, sb)
        torch.cuda.synchronize()
        tb1 = time.perf_counter()
        K.oscar_profile_enable(False)
        bms, bl = K.oscar_profile_read()
        bctx_np = btab[1].astype(np.int64)
        b_alg = int(bctx_np.sum()) * hkv * 512 + B * hq * 128 * 6
        b_main = bms / max(bl, 1)
        baseline = {
            "kv_tokens_per_s": float(bctx_np.sum() * nb / (tb1 - tb0)),
            "kernel": "decode_bf16",
            "kernel_us": round(b_main * 1e3, 2),
            "achieved_gbs": round(b_alg / (b_main * 1e-3) / 1e9, 1),
            "frac": round(b_alg / (b_main * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": b_alg,
            "splits": sb,
        }
        # plain copy of a known size (1 GiB read + 1 GiB written), for scaling
        # rocprofv3 FETCH_SIZE / WRITE_SIZE counters
        page_bytes = hkv * 8192
        n_copy = (1 << 30) // page_bytes
        cbuf = torch.zeros(2 * n_copy * page_bytes, dtype=torch.uint8, device="cuda")
        ccache = K.make_cache(None, 0, cbuf, 2 * n_copy)
        src = torch.arange(n_copy, dtype=torch.int32, device="cuda")
        K.oscar_copy_pages(bc.shape, ccache, 1, src, src + n_copy)
        torch.cuda.synchronize()
        del cbuf
        log(f"copy calibration: {n_copy} pages x {page_bytes} B = {n_copy * page_bytes} B read and written")
        log(f"bf16 baseline: decode_bf16 {b_main * 1e3:.1f} us, {baseline['achieved_gbs']} GB/s; "
            f"INT2/bf16 kernel time ratio {b_main / main_avg_ms:.2f}x")

    # ---- quant_write timed on its own: the workload's prefill chunk and a 16384-token chunk ----
    def time_write(ct, seed_req):
        dcc = DeviceCache(sh, r_k, r_v, tau_k, tau_v, ct // 16 + 1, 1)
        kb, vb = synth.kv_request_bf16(w, seed_req, 0, ct)
        kcd, vcd, scd = to_dev_bits(kb), to_dev_bits(vb), to_dev_i32(np.arange(ct, dtype=np.int32))
        for _ in range(3):
            K.oscar_quant_write(sh, dcc.layer, dcc.cache, kcd, vcd, scd)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in evs:
            a.record()
            K.oscar_quant_write(sh, dcc.layer, dcc.cache, kcd, vcd, scd)
            b.record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
        cbytes = ct * hkv * (2 * 128 * 2 + 2 * (32 + (128 // group) * mb))
        ops = 2.0 * WRITE_DIGIT_PAIRS * 128 * 128 * 2 * hkv * ct
        del dcc
        return {"chunk_tokens": ct, "us_median": round(us, 1), "tokens_per_s": ct / (us * 1e-6),
                "gbs": round(cbytes / (us * 1e-6) / 1e9, 1),
                "frac": round(cbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "int8_mfma_frac": round(ops / (us * 1e-6) / (INT8_PEAK_TOPS * 1e12), 4)}

    chunk_write = None
    if w.write_chunk:
        chunk_write = time_write(w.write_chunk, 200_000)
        log(f"write chunk of {w.write_chunk} tokens on its own: {chunk_write['us_median']} us median, "
            f"{chunk_write['gbs']} GB/s")
    write_16k = time_write(16384, 200_001)
    log(f"write chunk of 16384 tokens on its own: {write_16k['us_median']} us median, "
        f"{write_16k['tokens_per_s'] / 1e9:.3f} G tok/s, {write_16k['gbs']} GB/s ({write_16k['frac']:.1%} of HBM), "
        f"int8 MFMA {write_16k['int8_mfma_frac']:.1%} of peak")

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.no_cpu:
        import oracle as O
        import threadpoolctl
        cal = O.calibrate_layer(qc, kc, vc)
        cores = len(os.sched_getaffinity(0))
        blas = threadpoolctl.threadpool_info()
        blas_threads = max([b.get("num_threads", 1) for b in blas] or [1])
        done_tokens, spent, n_req = 0, 0.0, 0
        T_s = T_final
        while spent < args.cpu_seconds and n_req < B:
            kb, vb = synth.kv_request_bf16(w, n_req, 0, T_s)
            st_ = O.store_request(kb, vb, cal, group, w.sink, w.recent, scale_bits)
            qb = synth.q_decode_bf16(w, n_req)
            c0 = time.perf_counter()
            O.decode_attention(qb, st_, cal, group)
            spent += time.perf_counter() - c0
            done_tokens += T_s
            n_req += 1
        cpu = {"value": done_tokens / spent, "unit": "KV tokens/s", "cores": min(cores, blas_threads),
               "kind": "oracle",
               "sample": f"{n_req} of {B} requests x {T_s} tokens, all {hq} query heads: fp64 numpy decode "
                         f"attention over the stored INT2/bf16 cache ({spent:.1f} s)"}
        log(f"cpu oracle: {cpu['value']:.3e} tok/s on {cpu['cores']} threads")

    qw = None
    if qw_tokens:
        qw_ops = 2.0 * WRITE_DIGIT_PAIRS * 128 * 128 * 2 * hkv * qw_tokens
        qw = {"tokens_per_s": qw_tokens / qw_time, "ms_total": round(qw_time * 1e3, 3),
              "int8_mfma_frac": round(qw_ops / qw_time / (INT8_PEAK_TOPS * 1e12), 4),
              "gbs": round(qw_tokens * hkv * (2 * 128 * 2 + 2 * (32 + (128 // group) * mb)) / qw_time / 1e9, 1)}

    # stored bits per KV element at the final context (bf16 sink/recent + INT2 history)
    n_i2 = int2_tokens(T_final, w.sink, w.recent)
    hist_bits = 2.0 + 8 * mb / group           # codes + the (scale, zero) pair per group
    bits_per_element = (n_i2 * hist_bits + (T_final - n_i2) * 16.0) / T_final
    res = {
        "metric": "INT2 paged decode attention: KV tokens/s + achieved HBM GB/s (% of peak)",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f16 mfma, f32 acc",
        "data": "synthetic (seeded generator; calibration on synthetic activations)",
        "config": {"workload": w.name, "batch": B, "context": T_final, "n_q_heads": hq, "n_kv_heads": hkv,
                   "head_dim": 128, "group": group, "sink": w.sink, "recent": w.recent, "page_size": 16,
                   "scale_bits": scale_bits, "bits_per_element": round(bits_per_element, 4),
                   "splits_int2": si, "step": "unfused" if args.unfused else ("fused, host tables" if host_tables else "fused"),
                   "interleaved_writes": bool(iw), "cold": bool(flush is not None),
                   "decode_form": args.decode_form},
        "value_basis": value_basis,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_int2", "kernel_us": round(main_avg_ms * 1e3, 2),
                     "kernel_us_min": round(float(each_ms.min()) * 1e3, 2) if each_ms.size else None,
                     "kernel_us_median": round(float(np.median(each_ms)) * 1e3, 2) if each_ms.size else None,
                     "algorithmic_bytes_per_launch": int(alg),
                     "algorithmic_bytes_unique_per_launch": int(alg_unique),
                     "frac_unique": round(alg_unique / (main_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_step": int(alg_step),
                     # the KV tokens of a step over this kernel's own time (value counts the
                     # whole step: the prologue with its writes, the combine, the boundaries)
                     "kernel_kv_tokens_per_s": tokens / args.steps / (main_avg_ms * 1e-3)},
        "cpu_baseline": cpu,
        "settle": settle,
        "step_gpu_us": round(step_gpu_us, 1),
        "host_issue_us_per_step": round((t_issued - t0) / args.steps * 1e6, 2),
        "step_gpu_us_over": "timed steps" if step_ev_range.start == args.warmup else "warm-up steps",
        "cold_flush_mb": args.cold_flush_mb,
        "interleaved_write": interleaved,
        "write_chunk": chunk_write,
        "write_chunk_16k": write_16k,
        "bf16_baseline": baseline,
        "quant_write": qw,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
