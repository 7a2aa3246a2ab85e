"""Torch-side driver of the C ABI: a paged cache held in torch device tensors,
the smoke entry point and the benchmark.  Imports nothing from the oracle."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_int2_amd as K


def to_dev_bits(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device int16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def to_dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


class DeviceCache:
    """One layer's paged cache on the GPU plus its host pool bookkeeping."""

    def __init__(self, shape: K.Shape, r_k: np.ndarray, r_v: np.ndarray, tau_k, tau_v, n_int2_pages: int,
                 n_bf16_pages: int, fill: int = 0, prepare: bool = True):
        """fill: the byte every page starts with (0xFF makes each unwritten
        bf16 value and fp16 or FP8 scale/zero a NaN).  prepare: R's digits
        prepared once for the write calls (oscar_layer_prepare), else derived
        in every write work group."""
        self.shape = shape
        self.pool = K.Pool(shape, n_int2_pages, n_bf16_pages)
        ib = K.oscar_int2_block_bytes(shape)
        bb = K.oscar_bf16_block_bytes(shape)
        self.int2 = torch.full((max(n_int2_pages, 1) * shape.n_kv_heads * ib,), fill, dtype=torch.uint8,
                               device="cuda")
        self.bf16 = torch.full((max(n_bf16_pages, 1) * shape.n_kv_heads * bb,), fill, dtype=torch.uint8,
                               device="cuda")
        self.cache = K.make_cache(self.int2, n_int2_pages, self.bf16, n_bf16_pages)
        self.r_k = torch.from_numpy(np.ascontiguousarray(r_k, dtype=np.float32)).cuda()
        # r_v None: V arrives rotated (R_V folded into the model's projections)
        self.r_v = None if r_v is None else torch.from_numpy(np.ascontiguousarray(r_v, dtype=np.float32)).cuda()
        self.layer = K.make_layer(self.r_k, self.r_v, tau_k, tau_v)
        self.r_prep = None
        if prepare:
            self.r_prep = torch.empty(K.oscar_layer_prep_bytes(shape), dtype=torch.uint8, device="cuda")
            K.oscar_layer_prepare(shape, self.layer, self.r_prep)
            self.layer = K.make_layer(self.r_k, self.r_v, tau_k, tau_v, self.r_prep)
        self.int2_block = ib
        self.bf16_block = bb

    def new_seq(self):
        return K.oscar_seq_create(self.pool)

    def append(self, seq, k_bits: np.ndarray, v_bits: np.ndarray):
        """Grow `seq` by the tokens k_bits/v_bits [n, Hkv, d] (bf16 bits)."""
        n = k_bits.shape[0]
        i2, bf, a_s, a_d = K.oscar_seq_plan_append(self.pool, seq, n)
        if len(a_s):
            K.oscar_requant_from_bf16(self.shape, self.layer, self.cache, to_dev_i32(a_s), to_dev_i32(a_d))
        k = to_dev_bits(k_bits)
        v = to_dev_bits(v_bits)
        if np.any(i2 >= 0):
            K.oscar_quant_write(self.shape, self.layer, self.cache, k, v, to_dev_i32(i2))
        if np.any(bf >= 0):
            K.oscar_bf16_write(self.shape, self.cache, k, v, to_dev_i32(bf))

    def fork(self, parent):
        child, src, dst, kind = K.oscar_seq_fork(self.pool, parent)
        for kd in (0, 1):
            sel = kind == kd
            if np.any(sel):
                K.oscar_copy_pages(self.shape, self.cache, kd, to_dev_i32(src[sel]), to_dev_i32(dst[sel]))
        return child

    def tables(self, seqs, max_int2=None, max_bf16=None):
        hi = max(1, max((K.oscar_seq_length(s) + 15) // 16 for s in seqs)) if max_int2 is None else max_int2
        sp = (self.shape.sink + 15) // 16 + self.shape.recent // 16
        hb = max(1, sp) if max_bf16 is None else max_bf16
        i2, bf, ctx = K.oscar_block_tables(self.pool, seqs, hi, hb)
        return i2, bf, ctx

    def decode(self, seqs, q_bits: np.ndarray, splits_int2=0, splits_bf16=0, tables=None):
        """q_bits: [B, Hq, d] bf16 bits -> fp32 [B, Hq, d] (device)."""
        i2, bf, ctx = tables if tables is not None else self.tables(seqs)
        B = len(seqs)
        si = splits_int2 or K.oscar_decode_auto_splits(self.shape, B, i2.shape[1])
        sb = splits_bf16 or 4
        ws = torch.empty(K.oscar_decode_workspace_bytes(self.shape, B, si, sb), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, self.shape.n_q_heads, 128), dtype=torch.float32, device="cuda")
        K.oscar_decode_attn(self.shape, self.layer, self.cache, to_dev_bits(q_bits), to_dev_i32(i2), to_dev_i32(bf),
                            to_dev_i32(ctx), out, ws, si, sb)
        return out

    def int2_block_bytes_of(self, page: int, head: int) -> np.ndarray:
        if not (0 <= page < self.cache.n_int2_pages and 0 <= head < self.shape.n_kv_heads):
            raise IndexError(f"INT2 block ({page}, {head}) outside the pool")
        off = (page * self.shape.n_kv_heads + head) * self.int2_block
        return self.int2[off:off + self.int2_block].cpu().numpy()

    def bf16_block_bytes_of(self, page: int, head: int) -> np.ndarray:
        if not (0 <= page < self.cache.n_bf16_pages and 0 <= head < self.shape.n_kv_heads):
            raise IndexError(f"bf16 block ({page}, {head}) outside the pool")
        off = (page * self.shape.n_kv_heads + head) * self.bf16_block
        return self.bf16[off:off + self.bf16_block].cpu().numpy()


class BaselineCache:
    """All-bf16 paged cache for the baseline decode (position p -> bf16 page p/16)."""

    def __init__(self, shape: K.Shape, n_pages: int, max_context: int):
        # every position is a "sink" position: position p lives in bf16 logical page p/16
        self.shape = K.make_shape(head_dim=128, n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads,
                                  group=shape.group, sink=-(-max_context // 16) * 16, recent=0)
        self.pool = K.Pool(self.shape, 0, n_pages)
        bb = K.oscar_bf16_block_bytes(self.shape)
        self.bf16 = torch.zeros(max(n_pages, 1) * shape.n_kv_heads * bb, dtype=torch.uint8, device="cuda")
        self.cache = K.make_cache(None, 0, self.bf16, n_pages)

    def new_seq(self):
        return K.oscar_seq_create(self.pool)

    def append(self, seq, k_bits, v_bits):
        n = k_bits.shape[0]
        i2, bf, a_s, a_d = K.oscar_seq_plan_append(self.pool, seq, n)
        assert not np.any(i2 >= 0) and not len(a_s)
        K.oscar_bf16_write(self.shape, self.cache, to_dev_bits(k_bits), to_dev_bits(v_bits), to_dev_i32(bf))

    def tables(self, seqs):
        _, bf, ctx = K.oscar_block_tables(self.pool, seqs, 0, self.shape.sink // 16)
        return bf, ctx

    def decode(self, seqs, q_bits, splits=0, tables=None):
        bf, ctx = tables if tables is not None else self.tables(seqs)
        B = len(seqs)
        s = splits or K.oscar_decode_auto_splits(self.shape, B, bf.shape[1])
        ws = torch.empty(K.oscar_decode_workspace_bytes(self.shape, B, 1, s), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, self.shape.n_q_heads, 128), dtype=torch.float32, device="cuda")
        K.oscar_decode_attn_bf16_baseline(self.shape, self.cache, to_dev_bits(q_bits), to_dev_i32(bf),
                                          to_dev_i32(ctx), out, ws, s)
        return out
