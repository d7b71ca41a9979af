"""Thin ctypes binding of libmk.so (include/mk.h), same names as the C ABI.

Argument marshalling only: every step of the decode path runs in the HIP kernel.
PyTorch tensors are accepted wherever the C ABI takes a device pointer (their
data_ptr() is passed); streams are torch.cuda streams (their HIP handle is passed).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_ABI_VERSION = 2
MK_DESC_WORDS = 32
MK_STATIC_SCRATCH_BYTES = 16 << 20
MK_OK, MK_E_INVAL, MK_E_UNSUPPORTED, MK_E_NOMEM, MK_E_HIP, MK_E_STATE, MK_E_RANGE, MK_E_DEVICE = 0, -1, -2, -3, -4, -5, -6, -7
MK_DBG_DUMP_N = 1
MK_DBG_TIMESTAMPS = 2
MK_DBG_WIDE_GEMV = 4
MK_DBG_PAGE_WALK = 8
MK_DBG_DROP_SIGNAL = 16
MK_DBG_VALU_GEMV = 32
MK_DBG_COUNT_TASKS = 64
MK_DBG_MERGE_TASKS = 128
MK_DBGK_ROUTE_SEL, MK_DBGK_ROUTE_GATE, MK_DBGK_ROUTER_LOGITS, MK_DBGK_NORM_IN, MK_DBGK_COUNTERS, MK_DBGK_TASK_DONE = 1, 2, 3, 4, 5, 6
MK_DBGK_TIMESTAMPS = 7
MK_DBGK_PAGE_WALK = 8
MK_DBGK_SLOTS = 9
EXPORTS = ("mk_load_model", "mk_build_tasks", "mk_decode_step", "mk_mixed_step", "mk_decode_step_static", "mk_next_tokens", "mk_status", "mk_debug_set", "mk_debug_read",
           "mk_set_grid", "mk_free_model", "mk_last_error", "mk_plan_tasks")


class MkError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


class mk_model_desc(C.Structure):
    _fields_ = [("abi_version", C.c_int32)] + [(n, C.c_int32) for n in (
        "n_layers", "d_model", "n_q_heads", "n_kv_heads", "d_head", "n_experts", "top_k", "d_ffn", "vocab", "page_size",
        "max_batch", "max_pages_per_seq")] + [("n_pages", C.c_int64), ("rms_eps", C.c_float), ("rope_base", C.c_float),
                                               ("router_bias", C.c_void_p)]


class mk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p)] + [
        (n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "w_router", "w_gate", "w_up", "w_down")]


class mk_batch(C.Structure):
    _fields_ = [("batch", C.c_int32), ("seq_lens", C.c_void_p), ("first_of", C.c_void_p)]


_lib = None


def lib():
    """Load libmk.so; fails loudly if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.mk_load_model.argtypes = [vp, vp, C.POINTER(vp)]
        L.mk_build_tasks.argtypes = [vp, vp, vp, i64, C.POINTER(i64)]
        L.mk_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.mk_mixed_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.mk_decode_step_static.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.mk_next_tokens.argtypes = [vp, C.POINTER(vp)]
        L.mk_status.argtypes = [vp, vp]
        L.mk_debug_set.argtypes = [vp, C.c_uint32]
        L.mk_debug_read.argtypes = [vp, C.c_int, vp, i64]
        L.mk_set_grid.argtypes = [vp, i32]
        L.mk_free_model.argtypes = [vp]
        L.mk_last_error.argtypes = []
        L.mk_last_error.restype = C.c_char_p
        L.mk_plan_tasks.argtypes = [vp, vp, vp, i64, C.POINTER(i64), C.POINTER(i32)]
        for n in EXPORTS:
            if n != "mk_last_error":
                getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != MK_OK:
        raise MkError(rc, lib().mk_last_error().decode())
    return rc


def _ptr(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return C.c_void_p(x.data_ptr())
    if isinstance(x, np.ndarray):
        return x.ctypes.data_as(C.c_void_p)
    return C.c_void_p(int(x))


def _stream(s):
    if s is None:
        import torch

        s = torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream if hasattr(s, "cuda_stream") else int(s))


_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int]
        _hip.hipMemcpyAsync.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_void_p]
    return _hip


def read_device(ptr: int, nbytes: int, dtype=np.int32) -> np.ndarray:
    """Synchronous device-to-host copy of a raw device pointer (e.g. the buffer of mk_next_tokens)."""
    out = np.empty(nbytes // np.dtype(dtype).itemsize, dtype)
    rc = _hiprt().hipMemcpy(out.ctypes.data_as(C.c_void_p), C.c_void_p(ptr), nbytes, 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed ({rc})")
    return out


def make_desc(shape, max_batch, max_pages_per_seq, n_pages, router_bias=None):
    """Model descriptor from a shape object with the synthetic-model fields; keeps router_bias alive."""
    bias = None if router_bias is None else np.ascontiguousarray(router_bias, np.float32)
    d = mk_model_desc(MK_ABI_VERSION, shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                      shape.n_experts, shape.top_k, shape.d_ffn, shape.vocab, 16, max_batch, max_pages_per_seq, n_pages,
                      shape.rms_eps, shape.rope_base, None if bias is None else bias.ctypes.data)
    d._keep = bias
    return d


class Model:
    """Handle over mk_model*: mk_load_model / mk_build_tasks / mk_decode_step / mk_mixed_step / mk_next_tokens /
    mk_status / mk_debug_set / mk_debug_read / mk_set_grid / mk_free_model."""

    def __init__(self, desc: mk_model_desc, weights: dict):
        L = desc.n_layers
        self.desc = desc
        arrs = {}
        for k in ("attn_norm", "wq", "wk", "wv", "wo", "w_router", "w_gate", "w_up", "w_down"):
            t = weights[k]
            arrs[k] = (C.c_void_p * L)(*[t[l].data_ptr() for l in range(L)])
        self._keep = (weights, arrs)
        w = mk_weights(weights["embed"].data_ptr(), weights["lm_head"].data_ptr(), weights["final_norm"].data_ptr(),
                       *[C.cast(arrs[k], C.c_void_p) for k in ("attn_norm", "wq", "wk", "wv", "wo", "w_router", "w_gate", "w_up",
                                                               "w_down")])
        h = C.c_void_p()
        _check(lib().mk_load_model(C.byref(desc), C.byref(w), C.byref(h)))
        self.h = h
        self.B = None

    def mk_build_tasks(self, seq_lens, want_tasks=False, first_of=None):
        sl = np.ascontiguousarray(seq_lens, np.int32)
        fo = None if first_of is None else np.ascontiguousarray(first_of, np.int32)
        b = mk_batch(len(sl), sl.ctypes.data, None if fo is None else fo.ctypes.data)
        n = C.c_int64()
        if want_tasks:
            _check(lib().mk_build_tasks(self.h, C.byref(b), None, 0, C.byref(n)))
            out = np.empty((n.value, MK_DESC_WORDS), np.int32)
            _check(lib().mk_build_tasks(self.h, C.byref(b), out.ctypes.data_as(C.c_void_p), n.value, C.byref(n)))
        else:
            out = None
            _check(lib().mk_build_tasks(self.h, C.byref(b), None, 0, C.byref(n)))
        self.B = len(sl)
        self.n_tasks = n.value
        return out if want_tasks else n.value

    def mk_decode_step(self, tokens, seq_lens, page_tables, kv_pages, logits_out, stream=None):
        _check(lib().mk_decode_step(self.h, _ptr(tokens), _ptr(seq_lens), _ptr(page_tables), _ptr(kv_pages), _ptr(logits_out),
                                    _stream(stream)))

    def mk_decode_step_static(self, tokens, seq_lens, page_tables, kv_pages, logits_out, stream=None):
        _check(lib().mk_decode_step_static(self.h, _ptr(tokens), _ptr(seq_lens), _ptr(page_tables), _ptr(kv_pages),
                                           _ptr(logits_out), _stream(stream)))

    def mk_mixed_step(self, tokens, seq_lens, first_of, page_tables, kv_pages, logits_out, stream=None):
        _check(lib().mk_mixed_step(self.h, _ptr(tokens), _ptr(seq_lens), _ptr(first_of), _ptr(page_tables), _ptr(kv_pages),
                                   _ptr(logits_out), _stream(stream)))

    def mk_next_tokens(self):
        p = C.c_void_p()
        _check(lib().mk_next_tokens(self.h, C.byref(p)))
        return p.value

    def mk_status(self, stream=None):
        return _check(lib().mk_status(self.h, _stream(stream)))

    def mk_debug_set(self, flags):
        _check(lib().mk_debug_set(self.h, flags))

    def mk_debug_read(self, kind, shape, dtype):
        out = np.empty(shape, dtype)
        _check(lib().mk_debug_read(self.h, kind, out.ctypes.data_as(C.c_void_p), out.nbytes))
        return out

    def mk_set_grid(self, n):
        _check(lib().mk_set_grid(self.h, n))

    def mk_free_model(self):
        if self.h:
            _check(lib().mk_free_model(self.h))
            self.h = None

    def __del__(self):
        try:
            self.mk_free_model()
        except Exception:
            pass


def mk_plan_tasks(desc: mk_model_desc, seq_lens, first_of=None):
    sl = np.ascontiguousarray(seq_lens, np.int32)
    fo = None if first_of is None else np.ascontiguousarray(first_of, np.int32)
    b = mk_batch(len(sl), sl.ctypes.data, None if fo is None else fo.ctypes.data)
    n = C.c_int64()
    nc = C.c_int32()
    _check(lib().mk_plan_tasks(C.byref(desc), C.byref(b), None, 0, C.byref(n), C.byref(nc)))
    out = np.empty((n.value, MK_DESC_WORDS), np.int32)
    _check(lib().mk_plan_tasks(C.byref(desc), C.byref(b), out.ctypes.data_as(C.c_void_p), n.value, C.byref(n), C.byref(nc)))
    return out, nc.value
