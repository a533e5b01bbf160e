"""CPU oracle of the quantized MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never links or calls it, and it
shares no code with the GPU path.  The arithmetic lives in ``oracle.c`` (plain
single-threaded C, double precision); this module only marshals arguments.

Pinned by ``tests/test_oracle_pins.py``: every function below has at least one
pin that does not re-use the oracle's own formula (format tables from the OCP
specifications, torch's float8 decode, brute-force sorts, closed forms,
a dense fp64 reference on the tiny layer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same source built with OpenMP: oracle_ffn_combine runs the listed
# assignments on all host cores (timing of the CPU baseline only)
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")

FMT_NVFP4 = 1
FMT_Q6K = 2
FMT_Q8_0 = 3
FMT_IQ3G = 4
FMT_IQ1G = 5


def build(force: bool = True) -> str:
    for lib_path, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(lib_path):
            tmp = lib_path + ".tmp"
            cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
                   "-ffp-contract=off", *extra, _SRC, "-o", tmp, "-lm"]
            subprocess.check_call(cmd)
            os.replace(tmp, lib_path)
    return _LIB


class OracleExperts(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("fmt_down", ctypes.c_int32),
                ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("gate_ts", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p),
                ("up_ts", ctypes.c_void_p),
                ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p),
                ("down_ts", ctypes.c_void_p)]


_lib = None
_lib_omp = None


def lib(parallel: bool = False):
    """The oracle library; parallel=True: the OpenMP timing build."""
    global _lib, _lib_omp
    if parallel:
        if _lib_omp is None:
            if not os.path.exists(_LIB_OMP):
                build(force=False)
            _lib_omp = _load(_LIB_OMP)
        return _lib_omp
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _load(_LIB)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    vp, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    L.oracle_e2m1.restype = ctypes.c_double
    L.oracle_e2m1.argtypes = [u32]
    L.oracle_e4m3.restype = ctypes.c_double
    L.oracle_e4m3.argtypes = [u32]
    L.oracle_bf16.restype = ctypes.c_double
    L.oracle_bf16.argtypes = [ctypes.c_uint16]
    L.oracle_f16.restype = ctypes.c_double
    L.oracle_f16.argtypes = [ctypes.c_uint16]
    L.oracle_round_bf16.restype = ctypes.c_uint16
    L.oracle_round_bf16.argtypes = [ctypes.c_double]
    L.oracle_nvfp4_weight.restype = ctypes.c_double
    L.oracle_nvfp4_weight.argtypes = [vp, vp, ctypes.c_float, i64, i64, i64]
    L.oracle_q6k_weight.restype = ctypes.c_double
    L.oracle_q6k_weight.argtypes = [vp, i64, i64, i64]
    L.oracle_router_logits.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp]
    L.oracle_topk.argtypes = [vp, i64, i64, i64, i32, vp, vp]
    L.oracle_bucket.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp]
    L.oracle_hist.argtypes = [vp, i64, i32, i32, vp]
    L.oracle_expert.argtypes = [ctypes.POINTER(OracleExperts), i64, vp, vp]
    L.oracle_ffn_combine.argtypes = [ctypes.POINTER(OracleExperts), vp, i64, i64, vp, vp,
                                     vp, vp, i64, vp, vp]
    L.oracle_decode_nvfp4.argtypes = [vp, vp, ctypes.c_float, i64, i64, vp]
    L.oracle_decode_q6k.argtypes = [vp, i64, i64, vp]
    L.oracle_q8_0_weight.restype = ctypes.c_double
    L.oracle_q8_0_weight.argtypes = [vp, i64, i64, i64]
    L.oracle_decode_q8_0.argtypes = [vp, i64, i64, vp]
    L.oracle_iq3g_weight.restype = ctypes.c_double
    L.oracle_iq3g_weight.argtypes = [vp, i64, i64, i64]
    L.oracle_decode_iq3g.argtypes = [vp, i64, i64, vp]
    L.oracle_iq3g_grid.argtypes = [vp]
    L.oracle_iq1g_weight.restype = ctypes.c_double
    L.oracle_iq1g_weight.argtypes = [vp, i64, i64, i64]
    L.oracle_decode_iq1g.argtypes = [vp, i64, i64, vp]
    L.oracle_iq1g_grid.argtypes = [vp]
    L.oracle_expert_rows.argtypes = [ctypes.POINTER(OracleExperts), i64, vp, i64, vp]
    L.oracle_init.argtypes = []
    L.oracle_init()
    return L


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


# ---- formats -------------------------------------------------------------

def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e4m3(b: int) -> float:
    return lib().oracle_e4m3(b)


def bf16(bits: int) -> float:
    return lib().oracle_bf16(bits)


def f16(bits: int) -> float:
    return lib().oracle_f16(bits)


def round_bf16(v: float) -> int:
    return int(lib().oracle_round_bf16(v))


def decode_nvfp4(codes: np.ndarray, scales: np.ndarray, ts: float) -> np.ndarray:
    N = codes.shape[0]
    K = codes.shape[1] * 2
    out = np.empty((N, K), np.float64)
    lib().oracle_decode_nvfp4(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)),
                              ts, N, K, _p(out))
    return out


def decode_q6k(blocks: np.ndarray, K: int) -> np.ndarray:
    N = blocks.shape[0]
    out = np.empty((N, K), np.float64)
    lib().oracle_decode_q6k(_p(np.ascontiguousarray(blocks)), N, K, _p(out))
    return out


def decode_q8_0(blocks: np.ndarray, K: int) -> np.ndarray:
    """Q8_0-style rows [N][K/32*34] -> float64 [N][K] (d * q per 32-block)."""
    N = blocks.shape[0]
    out = np.empty((N, K), np.float64)
    lib().oracle_decode_q8_0(_p(np.ascontiguousarray(blocks)), N, K, _p(out))
    return out


def decode_iq3g(blocks: np.ndarray, K: int) -> np.ndarray:
    """IQ3-style grid rows [N][K/256*102] -> float64 [N][K]."""
    N = blocks.shape[0]
    out = np.empty((N, K), np.float64)
    lib().oracle_decode_iq3g(_p(np.ascontiguousarray(blocks)), N, K, _p(out))
    return out


def iq3g_grid() -> np.ndarray:
    """The oracle's 256-entry grid of the IQ3-style format, uint8 [256][4]."""
    out = np.empty((256, 4), np.uint8)
    lib().oracle_iq3g_grid(_p(out))
    return out


def decode_iq1g(blocks: np.ndarray, K: int) -> np.ndarray:
    """IQ1-style ternary-grid rows [N][K/256*46] -> float64 [N][K]."""
    N = blocks.shape[0]
    out = np.empty((N, K), np.float64)
    lib().oracle_decode_iq1g(_p(np.ascontiguousarray(blocks)), N, K, _p(out))
    return out


def iq1g_grid() -> np.ndarray:
    """The oracle's 1024-entry ternary grid of the IQ1-style format, int8 [1024][8]."""
    out = np.empty((1024, 8), np.int8)
    lib().oracle_iq1g_grid(_p(out))
    return out


# ---- layer steps ---------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None, order: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x, np.uint16)
    T, H = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_p(x), T, H, _p(np.ascontiguousarray(w_router, np.float32)),
                               _p(None if bias is None else np.ascontiguousarray(bias, np.float32)),
                               E, order, _p(out))
    return out


def topk(logits: np.ndarray, k: int, renormalize: int = 1):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().oracle_topk(_p(logits), T, E, k, renormalize, _p(idx), _p(w))
    return idx, w


def bucket(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, np.int32).reshape(-1)
    A = idx.size
    counts = np.empty(E, np.uint32)
    offsets = np.empty(E + 1, np.int32)
    sorted_asg = np.empty(A, np.int32)
    pos = np.empty(A, np.int32)
    active = np.empty(E, np.int32)
    n_active = np.zeros(1, np.int32)
    lib().oracle_bucket(_p(idx), A, E, _p(counts), _p(offsets), _p(sorted_asg), _p(pos),
                        _p(active), _p(n_active))
    return dict(counts=counts, offsets=offsets, sorted_asg=sorted_asg, asg_pos=pos,
                active=active[: int(n_active[0])].copy(), n_active=int(n_active[0]))


def hist(counts: np.ndarray, hist_in: np.ndarray, decay_shift: int, unit_shift: int) -> np.ndarray:
    h = np.ascontiguousarray(hist_in, np.uint32).copy()
    c = np.ascontiguousarray(counts, np.uint32)
    lib().oracle_hist(_p(c), c.size, decay_shift, unit_shift, _p(h))
    return h


def experts_struct(L):
    """OracleExperts view of a moegen.LayerWeights (keeps references alive)."""
    s = OracleExperts(L.E, L.H, L.I, L.fmt_down,
                      _p(L.gate_q), _p(L.gate_s), _p(L.gate_ts),
                      _p(L.up_q), _p(L.up_s), _p(L.up_ts),
                      _p(L.down_q), _p(L.down_s), _p(L.down_ts))
    s._keep = L
    return s


def expert(L, e: int, x_row: np.ndarray) -> np.ndarray:
    s = experts_struct(L)
    y = np.empty(L.H, np.float64)
    lib().oracle_expert(ctypes.byref(s), e, _p(np.ascontiguousarray(x_row, np.uint16)), _p(y))
    return y


def expert_rows(L, e: int, x_rows: np.ndarray) -> np.ndarray:
    """Expert e on each bf16 row of x_rows [n][H] -> float64 [n][H]; every row
    equals expert(L, e, row) bit for bit (the weights are decoded once)."""
    s = experts_struct(L)
    x_rows = np.ascontiguousarray(x_rows, np.uint16).reshape(-1, L.H)
    y = np.empty((x_rows.shape[0], L.H), np.float64)
    lib().oracle_expert_rows(ctypes.byref(s), e, _p(x_rows), x_rows.shape[0], _p(y))
    return y


def ffn_combine(L, x: np.ndarray, idx: np.ndarray, w: np.ndarray, residual=None,
                tokens=None, want_y: bool = False, parallel: bool = False):
    """Layer output bf16 bits [T][H] (rows of unlisted tokens are zero).
    parallel: the OpenMP build (same results, all host cores)."""
    s = experts_struct(L)
    x = np.ascontiguousarray(x, np.uint16)
    T = x.shape[0]
    k = idx.shape[1]
    out = np.zeros((T, L.H), np.uint16)
    y = np.zeros((T * k, L.H), np.float64) if want_y else None
    tok = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
    lib(parallel).oracle_ffn_combine(ctypes.byref(s), _p(x), T, k,
                             _p(np.ascontiguousarray(idx, np.int32)),
                             _p(np.ascontiguousarray(w, np.float32)),
                             _p(None if residual is None else np.ascontiguousarray(residual, np.uint16)),
                             _p(tok), 0 if tok is None else tok.size, _p(out), _p(y))
    return (out, y) if want_y else out


def route(x, L, order: int = 0):
    logits = router_logits(x, L.w_router, L.bias, order)
    idx, w = topk(logits, L.k, L.renormalize)
    return logits, idx, w


def layer(x, L, residual=None, tokens=None, parallel: bool = False):
    """Full layer: route, bucket, experts and combine for the given tokens
    (parallel: the experts on all host cores, same results)."""
    logits, idx, w = route(x, L)
    b = bucket(idx, L.E)
    out = ffn_combine(L, x, idx, w, residual, tokens, parallel=parallel)
    return dict(logits=logits, idx=idx, w=w, buckets=b, out=out)
