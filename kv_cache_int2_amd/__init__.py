"""Python binding of the OSCAR INT2 KV-cache library (liboscar.so, gfx950).

Argument marshalling only: every step of the path runs in the HIP library.
Device buffers are torch tensors (data_ptr); kernels are enqueued on torch's
current HIP stream.  The function names mirror the C ABI in include/oscar.h.
If the library has not been built, importing works but every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# OSCAR_LIB names another build of the same library (the host-sanitizer
# build liboscar_san.so is loaded this way by its test).
LIB_PATH = os.environ.get("OSCAR_LIB") or os.path.join(HERE, "liboscar.so")

OSCAR_OK, OSCAR_EINVAL, OSCAR_ENOMEM, OSCAR_EHIP, OSCAR_EUNSUPPORTED = 0, -1, -2, -3, -4
PAGE = 16


class OscarError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"oscar error {code}: {msg}")
        self.code = code


class Shape(C.Structure):
    _fields_ = [("head_dim", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("group", C.c_int32), ("sink", C.c_int32), ("recent", C.c_int32), ("page_size", C.c_int32),
                ("scale_bits", C.c_int32)]


class Layer(C.Structure):
    _fields_ = [("r_k", C.c_void_p), ("r_v", C.c_void_p), ("tau_k", C.c_float), ("tau_v", C.c_float),
                ("r_prep", C.c_void_p)]


class Cache(C.Structure):
    _fields_ = [("int2_pages", C.c_void_p), ("n_int2_pages", C.c_int64),
                ("bf16_pages", C.c_void_p), ("n_bf16_pages", C.c_int64)]


_lib = None
P = C.c_void_p
I32P = C.POINTER(C.c_int32)
I64P = C.POINTER(C.c_int64)

_SIGS = {
    "oscar_last_error": (C.c_char_p, []),
    "oscar_int2_block_bytes": (C.c_int64, [C.POINTER(Shape)]),
    "oscar_bf16_block_bytes": (C.c_int64, [C.POINTER(Shape)]),
    "oscar_calibrate_host": (C.c_int32, [C.POINTER(Shape), C.c_int64, P, P, P, C.c_double, C.c_double,
                                         P, P, P, P, P, P]),
    "oscar_calibrate_host_rotation": (C.c_int32, [C.POINTER(Shape), C.c_int32, C.c_int64, P, P, P, C.c_double,
                                                  C.c_double, P, P, P, P, P, P]),
    "oscar_pool_create": (C.c_int32, [C.POINTER(Shape), C.c_int64, C.c_int64, C.POINTER(P)]),
    "oscar_pool_destroy": (C.c_int32, [P]),
    "oscar_pool_free_pages": (C.c_int32, [P, I64P, I64P]),
    "oscar_seq_create": (C.c_int32, [P, C.POINTER(P)]),
    "oscar_seq_release": (C.c_int32, [P, P]),
    "oscar_seq_length": (C.c_int64, [P]),
    "oscar_seq_plan_append": (C.c_int32, [P, P, C.c_int64, P, P, P, P, I64P]),
    "oscar_seq_fork": (C.c_int32, [P, P, C.POINTER(P), P, P, P, I64P]),
    "oscar_block_tables": (C.c_int32, [P, P, C.c_int32, P, C.c_int32, P, C.c_int32, P]),
    "oscar_quant_write": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, P, P,
                                      C.c_int64, P]),
    "oscar_requant_from_bf16": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, P,
                                            C.c_int64, P]),
    "oscar_bf16_write": (C.c_int32, [C.POINTER(Shape), C.POINTER(Cache), P, P, P, C.c_int64, P]),
    "oscar_copy_pages": (C.c_int32, [C.POINTER(Shape), C.POINTER(Cache), C.c_int32, P, P, C.c_int64, P]),
    "oscar_decode_workspace_bytes": (C.c_size_t, [C.POINTER(Shape), C.c_int32, C.c_int32, C.c_int32]),
    "oscar_decode_attn": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, C.c_int32, P,
                                      C.c_int32, P, C.c_int32, P, C.c_int32, C.c_int32, P, P, C.c_size_t, P]),
    "oscar_decode_step": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, P, P, P,
                                      C.c_int32, P, C.c_int32, P, C.c_int32, P, C.c_int32, C.c_int32, P, P,
                                      C.c_size_t, P]),
    "oscar_decode_step_host_tables": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, P, P,
                                                  P, C.c_int32, P, C.c_int32, P, C.c_int32, P, C.c_int32,
                                                  C.c_int32, P, P, C.c_size_t, P]),
    "oscar_prefill_workspace_bytes": (C.c_size_t, [C.POINTER(Shape), C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "oscar_prefill_attn": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, C.c_int32,
                                       C.c_int32, P, C.c_int32, P, C.c_int32, P, C.c_int32, C.c_int32, P, P,
                                       C.c_size_t, P]),
    "oscar_decode_attn_noalloc": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), C.POINTER(Cache), P, C.c_int32,
                                              P, C.c_int32, P, C.c_int32, P, C.c_int32, C.c_int32, P, P]),
    "oscar_decode_noalloc_max_workspace_bytes": (C.c_size_t, []),
    "oscar_decode_attn_bf16_baseline": (C.c_int32, [C.POINTER(Shape), C.POINTER(Cache), P, C.c_int32, P,
                                                    C.c_int32, P, C.c_int32, P, P, C.c_size_t, P]),
    "oscar_decode_auto_splits": (C.c_int32, [C.POINTER(Shape), C.c_int32, C.c_int32]),
    "oscar_layer_prep_bytes": (C.c_size_t, [C.POINTER(Shape)]),
    "oscar_layer_prepare": (C.c_int32, [C.POINTER(Shape), C.POINTER(Layer), P, C.c_size_t, P]),
    "oscar_decode_set_small_grid": (C.c_int32, [C.c_int32]),
    "oscar_prefill_auto_splits": (C.c_int32, [C.POINTER(Shape), C.c_int32, C.c_int32, C.c_int32]),
    "oscar_plan_decode_step": (C.c_int32, [P, P, C.c_int32, P, P, P, P, P, P, P]),
    "oscar_profile_enable": (C.c_int32, [C.c_int32]),
    "oscar_profile_read": (C.c_int32, [C.POINTER(C.c_double), I64P]),
    "oscar_profile_read_each": (C.c_int32, [P, C.c_int64, C.POINTER(C.c_double), I64P]),
}
EXPORTED = tuple(_SIGS)


def lib():
    """The loaded liboscar.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OscarError(OSCAR_EUNSUPPORTED, f"{LIB_PATH} not built: run __graft_entry__.build()")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(code):
    if code != OSCAR_OK:
        raise OscarError(code, lib().oscar_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr() if t.numel() else None
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    return t


def _stream(stream=None):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def make_shape(head_dim=128, n_q_heads=1, n_kv_heads=1, group=32, sink=4, recent=128, page_size=PAGE,
               scale_bits=16) -> Shape:
    return Shape(head_dim, n_q_heads, n_kv_heads, group, sink, recent, page_size, scale_bits)


def make_layer(r_k, r_v, tau_k, tau_v, r_prep=None) -> Layer:
    """r_k, r_v: device fp32 tensors [n_kv, d, d]; r_prep: the prepared digits
    (oscar_layer_prepare) or None (all kept alive by the caller)."""
    return Layer(_ptr(r_k), _ptr(r_v), float(tau_k), float(tau_v), _ptr(r_prep))


def oscar_layer_prep_bytes(shape) -> int:
    return int(lib().oscar_layer_prep_bytes(C.byref(shape)))


def oscar_layer_prepare(shape, layer, prep, stream=None):
    """prep: device uint8 tensor of at least oscar_layer_prep_bytes(shape) bytes."""
    _check(lib().oscar_layer_prepare(C.byref(shape), C.byref(layer), _ptr(prep), prep.numel() * prep.element_size(),
                                     _stream(stream)))


def make_cache(int2_pages=None, n_int2_pages=0, bf16_pages=None, n_bf16_pages=0) -> Cache:
    return Cache(_ptr(int2_pages), int(n_int2_pages), _ptr(bf16_pages), int(n_bf16_pages))


def oscar_int2_block_bytes(shape: Shape) -> int:
    return int(lib().oscar_int2_block_bytes(C.byref(shape)))


def oscar_bf16_block_bytes(shape: Shape) -> int:
    return int(lib().oscar_bf16_block_bytes(C.byref(shape)))


ROTATION_OSCAR, ROTATION_IDENTITY, ROTATION_HADAMARD = 0, 1, 2
ROTATIONS = {"oscar": ROTATION_OSCAR, "identity": ROTATION_IDENTITY, "hadamard": ROTATION_HADAMARD}


def oscar_calibrate_host(shape: Shape, q, k, v, clip_pct_k=0.96, clip_pct_v=0.92, rotation="oscar"):
    """q: float32 numpy [n, Hq, d]; k, v: [n, Hkv, d].  Returns
    (r_k [Hkv,d,d] f32, r_v, eig_k [Hkv,d] f64, eig_v, tau_k, tau_v).
    rotation: "oscar", or the baselines "identity" / "hadamard"
    (oscar_calibrate_host_rotation)."""
    import numpy as np
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    n, hkv, d = k.shape
    r_k = np.empty((hkv, d, d), np.float32)
    r_v = np.empty_like(r_k)
    e_k = np.empty((hkv, d), np.float64)
    e_v = np.empty_like(e_k)
    tk, tv = C.c_float(), C.c_float()
    _check(lib().oscar_calibrate_host_rotation(C.byref(shape), ROTATIONS[rotation], n, q.ctypes.data,
                                               k.ctypes.data, v.ctypes.data, clip_pct_k, clip_pct_v,
                                               r_k.ctypes.data, r_v.ctypes.data, e_k.ctypes.data, e_v.ctypes.data,
                                               C.addressof(tk), C.addressof(tv)))
    return r_k, r_v, e_k, e_v, np.float32(tk.value), np.float32(tv.value)


class Pool:
    """Host bookkeeping of INT2 and bf16 page pools (oscar_pool_*)."""

    def __init__(self, shape: Shape, n_int2_pages: int, n_bf16_pages: int):
        self.shape = shape
        h = P()
        _check(lib().oscar_pool_create(C.byref(shape), n_int2_pages, n_bf16_pages, C.byref(h)))
        self.handle = h

    def free_pages(self):
        a, b = C.c_int64(), C.c_int64()
        _check(lib().oscar_pool_free_pages(self.handle, C.byref(a), C.byref(b)))
        return a.value, b.value

    def close(self):
        if self.handle:
            lib().oscar_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def oscar_seq_create(pool: Pool):
    h = P()
    _check(lib().oscar_seq_create(pool.handle, C.byref(h)))
    return h


def oscar_seq_release(pool: Pool, seq):
    _check(lib().oscar_seq_release(pool.handle, seq))


def oscar_seq_length(seq) -> int:
    return int(lib().oscar_seq_length(seq))


def oscar_seq_plan_append(pool: Pool, seq, n_new: int):
    """Returns numpy int32 arrays (int2_slots, bf16_slots, age_src, age_dst)."""
    import numpy as np
    i2 = np.empty(max(n_new, 1), np.int32)
    bf = np.empty(max(n_new, 1), np.int32)
    cap = max(n_new + pool.shape.recent, 1)
    a_s = np.empty(cap, np.int32)
    a_d = np.empty(cap, np.int32)
    na = C.c_int64()
    _check(lib().oscar_seq_plan_append(pool.handle, seq, n_new, i2.ctypes.data, bf.ctypes.data, a_s.ctypes.data,
                                       a_d.ctypes.data, C.byref(na)))
    return i2[:n_new], bf[:n_new], a_s[:na.value], a_d[:na.value]


def oscar_seq_fork(pool: Pool, parent):
    """Returns (child, copy_src, copy_dst, copy_kind) with numpy int32 arrays."""
    import numpy as np
    cap = 64 + pool.shape.recent // PAGE + 4
    src = np.empty(cap, np.int32)
    dst = np.empty(cap, np.int32)
    kind = np.empty(cap, np.int32)
    n = C.c_int64()
    child = P()
    _check(lib().oscar_seq_fork(pool.handle, parent, C.byref(child), src.ctypes.data, dst.ctypes.data,
                                kind.ctypes.data, C.byref(n)))
    return child, src[:n.value], dst[:n.value], kind[:n.value]


def oscar_block_tables(pool: Pool, seqs, max_int2_pages: int, max_bf16_pages: int):
    """Returns numpy (int2_bt [n, max_int2], bf16_bt [n, max_bf16], ctx_lens [n])."""
    import numpy as np
    n = len(seqs)
    arr = (P * max(n, 1))(*seqs)
    i2 = np.empty((n, max_int2_pages), np.int32)
    bf = np.empty((n, max_bf16_pages), np.int32)
    ctx = np.empty(n, np.int32)
    _check(lib().oscar_block_tables(pool.handle, arr, n, i2.ctypes.data if i2.size else None, max_int2_pages,
                                    bf.ctypes.data if bf.size else None, max_bf16_pages, ctx.ctypes.data))
    return i2, bf, ctx


def oscar_quant_write(shape, layer, cache, k_bf16, v_bf16, int2_slots, n=None, stream=None):
    n = int2_slots.numel() if n is None else n
    _check(lib().oscar_quant_write(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(k_bf16), _ptr(v_bf16),
                                   _ptr(int2_slots), n, _stream(stream)))


def oscar_requant_from_bf16(shape, layer, cache, src_bf16_slots, dst_int2_slots, n=None, stream=None):
    n = src_bf16_slots.numel() if n is None else n
    _check(lib().oscar_requant_from_bf16(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(src_bf16_slots),
                                         _ptr(dst_int2_slots), n, _stream(stream)))


def oscar_bf16_write(shape, cache, k_bf16, v_bf16, bf16_slots, n=None, stream=None):
    n = bf16_slots.numel() if n is None else n
    _check(lib().oscar_bf16_write(C.byref(shape), C.byref(cache), _ptr(k_bf16), _ptr(v_bf16), _ptr(bf16_slots), n,
                                  _stream(stream)))


def oscar_copy_pages(shape, cache, kind, src_pages, dst_pages, n=None, stream=None):
    n = src_pages.numel() if n is None else n
    _check(lib().oscar_copy_pages(C.byref(shape), C.byref(cache), kind, _ptr(src_pages), _ptr(dst_pages), n,
                                  _stream(stream)))


def oscar_decode_workspace_bytes(shape, batch, splits_int2=0, splits_bf16=0) -> int:
    return int(lib().oscar_decode_workspace_bytes(C.byref(shape), batch, splits_int2, splits_bf16))


def oscar_decode_auto_splits(shape, batch, max_int2_pages) -> int:
    return int(lib().oscar_decode_auto_splits(C.byref(shape), batch, max_int2_pages))


def oscar_decode_set_small_grid(mode: int) -> int:
    return int(lib().oscar_decode_set_small_grid(mode))


def oscar_prefill_auto_splits(shape, batch, max_int2_pages, chunk) -> int:
    return int(lib().oscar_prefill_auto_splits(C.byref(shape), batch, max_int2_pages, chunk))


def oscar_decode_attn(shape, layer, cache, q, int2_bt, bf16_bt, ctx_lens, out, workspace, splits_int2=0,
                      splits_bf16=0, stream=None):
    batch = q.shape[0]
    _check(lib().oscar_decode_attn(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(q), batch, _ptr(int2_bt),
                                   int2_bt.shape[1], _ptr(bf16_bt), bf16_bt.shape[1], _ptr(ctx_lens), splits_int2,
                                   splits_bf16, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def oscar_decode_step(shape, layer, cache, k_new, v_new, step_slots, q, int2_bt, bf16_bt, ctx_lens, out, workspace,
                      splits_int2=0, splits_bf16=0, stream=None):
    """Fused decode step: step_slots int32 [4][batch] rows = new token's INT2
    slot, new token's bf16 slot, leaving token's bf16 source, its INT2 target."""
    batch = q.shape[0]
    _check(lib().oscar_decode_step(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(k_new), _ptr(v_new),
                                   _ptr(step_slots), _ptr(q), batch, _ptr(int2_bt), int2_bt.shape[1], _ptr(bf16_bt),
                                   bf16_bt.shape[1], _ptr(ctx_lens), splits_int2, splits_bf16, _ptr(out),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_decode_step_host_tables(shape, layer, cache, k_new, v_new, step_slots, q, int2_bt, bf16_bt, ctx_lens,
                                  out, workspace, splits_int2=0, splits_bf16=0, stream=None):
    """oscar_decode_step with step_slots int32 [4][batch] and ctx_lens int32
    [batch] as host numpy arrays (read during the call; batch <= 64)."""
    batch = q.shape[0]
    slots = np.ascontiguousarray(step_slots, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if slots.shape != (4, batch) or ctx.shape != (batch,):
        raise ValueError(f"step_slots must be [4][{batch}] and ctx_lens [{batch}] (got {slots.shape}, {ctx.shape})")
    _check(lib().oscar_decode_step_host_tables(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(k_new),
                                               _ptr(v_new), _ptr(slots), _ptr(q), batch, _ptr(int2_bt),
                                               int2_bt.shape[1], _ptr(bf16_bt), bf16_bt.shape[1], _ptr(ctx),
                                               splits_int2, splits_bf16, _ptr(out), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_prefill_workspace_bytes(shape, batch, chunk, splits_int2=0, splits_bf16=0) -> int:
    return int(lib().oscar_prefill_workspace_bytes(C.byref(shape), batch, chunk, splits_int2, splits_bf16))


def oscar_prefill_attn(shape, layer, cache, q, int2_bt, bf16_bt, ctx_lens, out, workspace, splits_int2=0,
                       splits_bf16=0, stream=None):
    """q: device bf16 bits [batch, C, Hq, d]; out: fp32 [batch, C, Hq, d]."""
    batch, chunk = q.shape[0], q.shape[1]
    _check(lib().oscar_prefill_attn(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(q), batch, chunk,
                                    _ptr(int2_bt), int2_bt.shape[1], _ptr(bf16_bt), bf16_bt.shape[1],
                                    _ptr(ctx_lens), splits_int2, splits_bf16, _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


def oscar_decode_attn_noalloc(shape, layer, cache, q, int2_bt, bf16_bt, ctx_lens, out, splits_int2=0, splits_bf16=0,
                              stream=None):
    batch = q.shape[0]
    _check(lib().oscar_decode_attn_noalloc(C.byref(shape), C.byref(layer), C.byref(cache), _ptr(q), batch,
                                           _ptr(int2_bt), int2_bt.shape[1], _ptr(bf16_bt), bf16_bt.shape[1],
                                           _ptr(ctx_lens), splits_int2, splits_bf16, _ptr(out), _stream(stream)))


def oscar_decode_noalloc_max_workspace_bytes() -> int:
    return int(lib().oscar_decode_noalloc_max_workspace_bytes())


def oscar_decode_attn_bf16_baseline(shape, cache, q, bf16_bt, ctx_lens, out, workspace, splits=0, stream=None):
    batch = q.shape[0]
    _check(lib().oscar_decode_attn_bf16_baseline(C.byref(shape), C.byref(cache), _ptr(q), batch, _ptr(bf16_bt),
                                                 bf16_bt.shape[1], _ptr(ctx_lens), splits, _ptr(out), _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)))


class DecodeStepPlanner:
    """oscar_plan_decode_step with reusable host arrays (pinned when torch
    can provide them), one call per decode step for the whole batch."""

    def __init__(self, pool: Pool, seqs):
        import numpy as np
        self.pool = pool
        self.n = len(seqs)
        self.arr = (P * max(self.n, 1))(*seqs)
        self.buf = np.zeros((5, max(self.n, 1)), np.int32)   # int2, bf16, age_src, age_dst, ctx
        self.n_age = C.c_int32()
        self.changed = C.c_int32()
        # the arguments never change (buf is reused): marshalled once
        b = self.buf
        self._fn = lib().oscar_plan_decode_step
        self._args = (self.pool.handle, self.arr, self.n, b[0].ctypes.data, b[1].ctypes.data, b[2].ctypes.data,
                      b[3].ctypes.data, C.byref(self.n_age), b[4].ctypes.data, C.byref(self.changed))

    def step(self):
        _check(self._fn(*self._args))
        return self.n_age.value, bool(self.changed.value)


def oscar_profile_enable(on: bool):
    _check(lib().oscar_profile_enable(1 if on else 0))


def oscar_profile_read():
    ms, n = C.c_double(), C.c_int64()
    _check(lib().oscar_profile_read(C.byref(ms), C.byref(n)))
    return ms.value, n.value


def oscar_profile_read_each(cap: int = 1 << 16):
    """(total ms, launch count, per-launch ms as a float32 array of the first cap launches)."""
    import numpy as np
    each = np.zeros(max(cap, 1), np.float32)
    ms, n = C.c_double(), C.c_int64()
    _check(lib().oscar_profile_read_each(each.ctypes.data, cap, C.byref(ms), C.byref(n)))
    return ms.value, n.value, each[:min(n.value, cap)].copy()
