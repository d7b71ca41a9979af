"""Seeded synthetic inputs: Python binding of libsynth_host.so / libsynth_dev.so.

Every value is a pure function of (seed, stream, logical index) (synth_core.h),
so the host copies used by the CPU oracle and the device copies used by the GPU
path hold identical bytes.  This module holds none of the decode method's
arithmetic; it only produces inputs.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Stream kinds, mirroring synth_core.h.
EMBED, LM_HEAD, WQ, WK, WV, WO, WROUTER, WGATE, WUP, WDOWN, NORM = range(1, 12)
KV_POS_SPAN = 1 << 20


def weight_stream(kind: int, layer: int) -> int:
    return (kind << 32) | (layer & 0xFFFFFFFF)


def build_host(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           os.path.join(_HERE, "synth.c"), "-o", HOST_LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(HOST_LIB + ".tmp", HOST_LIB)


def build_dev(verbose=False):
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "synth_dev.hip"), "-o", DEV_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL if not verbose else None)
    os.replace(DEV_LIB + ".tmp", DEV_LIB)


_host = None
_dev = None


def host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        L = C.CDLL(HOST_LIB)
        vp, i64, u64, i32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_int32
        L.synth_table_build.argtypes = [C.c_double, vp, vp, vp]
        L.synth_table_build.restype = C.c_int
        L.synth_fill_bf16.argtypes = [vp, i64, u64, u64, u64, vp, vp]
        L.synth_fill_kv_paged.argtypes = [vp, C.c_int, C.c_int, i64, C.c_int, C.c_int, C.c_int, vp, i64, C.c_int, i64, i64, u64, vp, vp]
        L.synth_fill_kv_paged.restype = C.c_int
        L.synth_u64_fill.argtypes = [u64, u64, u64, i64, vp]
        L.synth_splitmix64.argtypes = [u64, i64, vp]
        L.synth_token.argtypes = [u64, C.c_int, C.c_int]
        L.synth_token.restype = i32
        L.synth_loguniform_ints.argtypes = [u64, u64, C.c_int, i64, i64, vp]
        L.synth_permutation.argtypes = [u64, u64, C.c_int, vp]
        L.synth_skew_bias.argtypes = [u64, C.c_int, C.c_double, vp]
        _host = L
    return _host


def dev():
    """The device fill library; it must have been built (``__graft_entry__.build()``)."""
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is missing: run __graft_entry__.build() first")
        L = C.CDLL(DEV_LIB)
        vp, i64, u64 = C.c_void_p, C.c_int64, C.c_uint64
        L.synth_dev_fill_bf16.argtypes = [vp, i64, u64, u64, u64, vp, vp, vp]
        L.synth_dev_fill_bf16.restype = C.c_int
        L.synth_dev_fill_kv_paged.argtypes = [vp, C.c_int, C.c_int, i64, C.c_int, C.c_int, C.c_int, vp, C.c_int, i64, i64, u64, vp, vp,
                                              vp, vp]
        L.synth_dev_fill_kv_paged.restype = C.c_int
        _dev = L
    return _dev


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


class Table:
    """Inverse-CDF tables of N(0, sigma) rounded to BF16 (host arrays; device copies on demand)."""

    _cache: dict = {}

    def __init__(self, sigma: float):
        self.sigma = sigma
        self.thr = np.zeros(0x7F81, np.uint64)
        self.guide = np.zeros(1 << 16, np.uint16)
        n = C.c_int32(0)
        rc = host().synth_table_build(sigma, _p(self.thr), _p(self.guide), C.byref(n))
        if rc:
            raise ValueError(f"synth_table_build rc={rc}")
        self.n = n.value
        self.thr = self.thr[: self.n].copy()
        self._dev = {}

    @classmethod
    def get(cls, sigma: float) -> "Table":
        if sigma not in cls._cache:
            cls._cache[sigma] = Table(sigma)
        return cls._cache[sigma]

    def device(self, device="cuda"):
        import torch

        key = str(device)
        if key not in self._dev:
            thr = torch.from_numpy(self.thr.view(np.int64).copy()).to(device)
            guide = torch.from_numpy(self.guide.view(np.int16).copy()).to(device)
            self._dev[key] = (thr, guide)
        return self._dev[key]


def fill_bf16_host(n: int, seed: int, stream: int, index0: int = 0, sigma: float = 0.02) -> np.ndarray:
    t = Table.get(sigma)
    out = np.empty(int(n), np.uint16)
    host().synth_fill_bf16(_p(out), int(n), seed, stream, index0, _p(t.thr), _p(t.guide))
    return out


def fill_bf16_dev(tensor, seed: int, stream: int, index0: int = 0, sigma: float = 0.02):
    """Fill a contiguous 2-byte device tensor with the same values fill_bf16_host gives."""
    import torch

    assert tensor.is_cuda and tensor.is_contiguous() and tensor.element_size() == 2
    thr, guide = Table.get(sigma).device(tensor.device)
    s = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = dev().synth_dev_fill_bf16(C.c_void_p(tensor.data_ptr()), tensor.numel(), seed, stream, index0, C.c_void_p(thr.data_ptr()),
                                   C.c_void_p(guide.data_ptr()), C.c_void_p(s))
    if rc:
        raise RuntimeError(f"synth_dev_fill_bf16 rc={rc}")
    return tensor


def fill_kv_host(kv: np.ndarray, layer0: int, n_kv_heads: int, d_head: int, page_size: int, page_table, seq_id: int, pos0: int,
                 pos1: int, seed: int, sigma: float = 1.0):
    """kv: uint16 [n_layers_buf][n_pages][2][Hkv][page_size][dh], filled in place."""
    assert kv.dtype == np.uint16 and kv.flags.c_contiguous and kv.ndim == 6
    t = Table.get(sigma)
    pt = np.ascontiguousarray(page_table, np.int32)
    rc = host().synth_fill_kv_paged(_p(kv), kv.shape[0], layer0, kv.shape[1], n_kv_heads, d_head, page_size, _p(pt), pt.shape[0],
                                    seq_id, int(pos0), int(pos1), seed, _p(t.thr), _p(t.guide))
    if rc:
        raise ValueError(f"synth_fill_kv_paged rc={rc}")


def fill_kv_dev(kv, n_layers_buf: int, layer0: int, n_pages: int, n_kv_heads: int, d_head: int, page_size: int, page_table_dev,
                seq_id: int, pos0: int, pos1: int, seed: int, sigma: float = 1.0, bad=None):
    import torch

    thr, guide = Table.get(sigma).device(kv.device)
    s = torch.cuda.current_stream(kv.device).cuda_stream
    rc = dev().synth_dev_fill_kv_paged(C.c_void_p(kv.data_ptr()), n_layers_buf, layer0, n_pages, n_kv_heads, d_head, page_size,
                                       C.c_void_p(page_table_dev.data_ptr()), seq_id, int(pos0), int(pos1), seed,
                                       C.c_void_p(thr.data_ptr()), C.c_void_p(guide.data_ptr()),
                                       C.c_void_p(bad.data_ptr() if bad is not None else 0), C.c_void_p(s))
    if rc:
        raise RuntimeError(f"synth_dev_fill_kv_paged rc={rc}")


def splitmix64(state: int, n: int) -> np.ndarray:
    out = np.empty(int(n), np.uint64)
    host().synth_splitmix64(state, int(n), _p(out))
    return out


def u64(seed: int, stream: int, index0: int, n: int) -> np.ndarray:
    out = np.empty(int(n), np.uint64)
    host().synth_u64_fill(seed, stream, index0, int(n), _p(out))
    return out


def u01(seed: int, stream: int, index0: int, n: int) -> np.ndarray:
    return (u64(seed, stream, index0, n) >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def token(seed: int, seq: int, vocab: int) -> int:
    return int(host().synth_token(seed, seq, vocab))


def loguniform_ints(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, np.int64)
    host().synth_loguniform_ints(seed, stream, n, lo, hi, _p(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    host().synth_permutation(seed, stream, n, _p(out))
    return out


def skew_bias(seed: int, n_experts: int, scale: float = 1.5) -> np.ndarray:
    out = np.empty(n_experts, np.float32)
    host().synth_skew_bias(seed, n_experts, scale, _p(out))
    return out
