"""ctypes binding of the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only callers.  The GPU path never imports
this module.  What each function computes, and the passages of the pages it
follows, is stated in oracle.h.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (plain IEEE arithmetic, OpenMP)."""
    import subprocess

    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(_HERE, "oracle.c"), "-o", LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class OrDims(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "d_head", "n_experts",
                                         "top_k", "d_ffn", "vocab", "page_size")] + [
        ("rms_eps", C.c_double), ("rope_base", C.c_double)]


class OrLayerW(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wq", C.c_void_p), ("wk", C.c_void_p), ("wv", C.c_void_p),
                ("wo", C.c_void_p), ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p)]


_lib = None


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().or_num_threads())


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, d = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        L.or_matvec.argtypes = [vp, i64, i64, vp, vp]
        L.or_rmsnorm.argtypes = [vp, vp, C.c_int, d, vp]
        L.or_rope.argtypes = [vp, C.c_int, C.c_int, i64, d]
        L.or_attention.argtypes = [vp, vp, vp, i64, vp, i64, i64, vp]
        L.or_attention.restype = C.c_int
        L.or_router.argtypes = [vp, vp, vp, C.c_int, C.c_int, C.c_int, vp, vp, vp]
        L.or_expert.argtypes = [vp, vp, vp, vp, C.c_int, C.c_int, vp]
        L.or_layer.argtypes = [vp, vp, C.c_int, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        L.or_layer.restype = C.c_int
        L.or_embed.argtypes = [vp, vp, vp, C.c_int, vp]
        L.or_embed.restype = C.c_int
        L.or_head.argtypes = [vp, vp, C.c_int, vp, vp, vp, vp]
        L.or_decode_step.argtypes = [vp, vp, vp, vp, vp, C.c_int, vp, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp]
        L.or_decode_step.restype = C.c_int
        L.or_num_threads.argtypes = []
        L.or_num_threads.restype = C.c_int
        L.or_f32_to_bf16.argtypes = [C.c_float]
        L.or_f32_to_bf16.restype = C.c_uint16
        L.or_bf16_to_f32.argtypes = [C.c_uint16]
        L.or_bf16_to_f32.restype = C.c_float
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


@dataclass
class Dims:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    d_head: int
    n_experts: int
    top_k: int
    d_ffn: int
    vocab: int
    page_size: int = 16
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    def c(self) -> OrDims:
        return OrDims(self.n_layers, self.d_model, self.n_q_heads, self.n_kv_heads, self.d_head, self.n_experts,
                      self.top_k, self.d_ffn, self.vocab, self.page_size, self.rms_eps, self.rope_base)


def matvec(W, x):
    W, x = _u16(W), _f32(x)
    y = np.empty(W.shape[0], np.float32)
    lib().or_matvec(_p(W), W.shape[0], W.shape[1], _p(x), _p(y))
    return y


def rmsnorm(x, gamma, eps=1e-6):
    x, gamma = _f32(x), _u16(gamma)
    out = np.empty_like(x)
    lib().or_rmsnorm(_p(x), _p(gamma), x.shape[-1], eps, _p(out))
    return out


def rope(v, pos, base=10000.0):
    """v: [n_heads][d_head] float32, rotated copy returned."""
    v = _f32(v).copy()
    lib().or_rope(_p(v), v.shape[0], v.shape[1], int(pos), base)
    return v


def attention(D: Dims, q, kv_layer, page_table, n_ctx):
    q, kv_layer = _f32(q), _u16(kv_layer)
    pt = np.ascontiguousarray(page_table, np.int32)
    out = np.empty((D.n_q_heads, D.d_head), np.float32)
    dc = D.c()
    rc = lib().or_attention(C.byref(dc), _p(q), _p(kv_layer), kv_layer.shape[0], _p(pt), pt.shape[0], int(n_ctx), _p(out))
    if rc:
        raise ValueError(f"or_attention rc={rc}")
    return out


def router(n, w_router, k, bias=None):
    n, w = _f32(n), _u16(w_router)
    E = w.shape[0]
    sel = np.empty(k, np.int32)
    gate = np.empty(k, np.float32)
    logits = np.empty(E, np.float32)
    b = None if bias is None else _f32(bias)
    lib().or_router(_p(n), _p(w), _p(b), E, w.shape[1], k, _p(sel), _p(gate), _p(logits))
    return sel, gate, logits


def expert(n, wg, wu, wd):
    n, wg, wu, wd = _f32(n), _u16(wg), _u16(wu), _u16(wd)
    y = np.empty(wd.shape[0], np.float32)
    lib().or_expert(_p(n), _p(wg), _p(wu), _p(wd), wg.shape[1], wg.shape[0], _p(y))
    return y


class LayerWeights:
    """Keeps the numpy arrays of one layer alive and exposes the C struct.

    experts: dict e -> (w_gate [F][d], w_up [F][d], w_down [d][F]); experts not in the
    dict are passed as NULL (the oracle fails loudly if it selects one)."""

    def __init__(self, attn_norm, wq, wk, wv, wo, w_router, experts: dict, E: int, router_bias=None):
        self.arrs = [_u16(attn_norm), _u16(wq), _u16(wk), _u16(wv), _u16(wo), _u16(w_router)]
        self.bias = None if router_bias is None else _f32(router_bias)
        self.exp = {e: tuple(_u16(a) for a in t) for e, t in experts.items()}
        ptrs = [(C.c_void_p * E)() for _ in range(3)]
        for e, t in self.exp.items():
            for i in range(3):
                ptrs[i][e] = t[i].ctypes.data
        self.ptrs = ptrs
        a = self.arrs
        self.c = OrLayerW(a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data, a[3].ctypes.data, a[4].ctypes.data,
                          a[5].ctypes.data, None if self.bias is None else self.bias.ctypes.data,
                          C.cast(ptrs[0], C.c_void_p), C.cast(ptrs[1], C.c_void_p), C.cast(ptrs[2], C.c_void_p))


def layer(D: Dims, W: LayerWeights, pos, page_tables, kv_layer, x, sel_force=None):
    """One parallel layer for B tokens; updates kv_layer (uint16, in place) and returns the new x and diagnostics."""
    x = _f32(x).copy()
    B = x.shape[0]
    pos = np.ascontiguousarray(pos, np.int64)
    pt = np.ascontiguousarray(page_tables, np.int32)
    assert kv_layer.dtype == np.uint16 and kv_layer.flags.c_contiguous
    k, d, E = D.top_k, D.d_model, D.n_experts
    sel = np.empty((B, k), np.int32)
    gate = np.empty((B, k), np.float32)
    n = np.empty((B, d), np.float32)
    a = np.empty((B, d), np.float32)
    m = np.empty((B, d), np.float32)
    lg = np.empty((B, E), np.float32)
    sf = None if sel_force is None else np.ascontiguousarray(sel_force, np.int32)
    dc = D.c()
    rc = lib().or_layer(C.byref(dc), C.byref(W.c), B, _p(pos), _p(pt), pt.shape[1], _p(kv_layer), kv_layer.shape[0], _p(x),
                        _p(sf), _p(sel), _p(gate), _p(n), _p(a), _p(m), _p(lg))
    if rc:
        raise ValueError(f"or_layer rc={rc}")
    return x, dict(sel=sel, gate=gate, n=n, attn=a, moe=m, router_logits=lg)


def embed(D: Dims, E_w, tokens):
    tokens = np.ascontiguousarray(tokens, np.int32)
    x = np.empty((tokens.shape[0], D.d_model), np.float32)
    dc = D.c()
    if lib().or_embed(C.byref(dc), _p(_u16(E_w)), _p(tokens), tokens.shape[0], _p(x)):
        raise ValueError("token out of range")
    return x


def head(D: Dims, x, final_norm, lm_head):
    x = _f32(x)
    B = x.shape[0]
    logits = np.empty((B, D.vocab), np.float32)
    nxt = np.empty(B, np.int32)
    dc = D.c()
    lib().or_head(C.byref(dc), _p(x), B, _p(_u16(final_norm)), _p(_u16(lm_head)), _p(logits), _p(nxt))
    return logits, nxt


def f32_to_bf16(a):
    """Round-to-nearest-even fp32 -> BF16 bit patterns (vectorised; same rule as or_f32_to_bf16)."""
    a = _f32(a)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
