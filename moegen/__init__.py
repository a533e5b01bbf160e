"""Seeded synthetic inputs for the quantized MoE layer.

Holds none of the layer's arithmetic: it writes activations, router weights,
router biases and block-quantized expert weights (NVFP4, Q6_K-style) as bytes
that both the oracle and the GPU library read.  The C source is ``moegen.c``;
the shared library is built in-tree on first use (``build()``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moegen.c")
_LIB = os.path.join(_HERE, "libmoegen.so")

FMT_NVFP4 = 1
FMT_Q6K = 2
FMT_Q8_0 = 3
FMT_IQ3G = 4
FMT_IQ1G = 5

# stream tags
TAG_X = 1
TAG_ROUTER = 2
TAG_BIAS = 3
TAG_GATE = 4
TAG_UP = 5
TAG_DOWN = 6
TAG_RESID = 7
TAG_PERM = 8


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        L.moegen_key.restype = u64
        L.moegen_key.argtypes = [u64, u64, u64, u64]
        L.moegen_draw.restype = u64
        L.moegen_draw.argtypes = [u64, u64]
        for name in ("moegen_normal_f64", "moegen_normal_f32", "moegen_normal_bf16"):
            getattr(L, name).argtypes = [u64, i64, dbl, vp]
            getattr(L, name).restype = None
        L.moegen_quant_nvfp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.moegen_quant_q6k.argtypes = [vp, i64, i64, vp]
        L.moegen_nvfp4_normal.argtypes = [u64, i64, i64, dbl, vp, vp, vp, vp]
        L.moegen_q6k_normal.argtypes = [u64, i64, i64, dbl, vp, vp]
        L.moegen_quant_q8_0.argtypes = [vp, i64, i64, vp]
        L.moegen_q8_0_normal.argtypes = [u64, i64, i64, dbl, vp, vp]
        L.moegen_quant_iq3g.argtypes = [vp, i64, i64, vp]
        L.moegen_iq3g_normal.argtypes = [u64, i64, i64, dbl, vp, vp]
        L.moegen_quant_iq1g.argtypes = [vp, i64, i64, vp]
        L.moegen_iq1g_normal.argtypes = [u64, i64, i64, dbl, vp, vp]
        L.moegen_permutation.argtypes = [u64, i32, vp]
        L.moegen_zipf_bias.argtypes = [u64, i32, dbl, dbl, vp, vp]
        L.moegen_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def key(seed: int, tag: int, layer: int = 0, step: int = 0) -> int:
    return int(lib().moegen_key(seed, tag, layer, step))


def normal_f64(k: int, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().moegen_normal_f64(k, n, std, _p(out))
    return out


def normal_f32(k: int, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().moegen_normal_f32(k, n, std, _p(out))
    return out


def normal_bf16(k: int, n: int, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16), rounded to nearest even from fp32."""
    out = np.empty(n, np.uint16)
    lib().moegen_normal_bf16(k, n, std, _p(out))
    return out


def quant_nvfp4(W: np.ndarray):
    """fp32 [N][K] -> (codes u8 [N][K/2], scales u8 [N][K/16], ts float)."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 16 == 0
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, K // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    lib().moegen_quant_nvfp4(_p(W), N, K, _p(codes), _p(scales), _p(ts))
    return codes, scales, float(ts[0])


def quant_q6k(W: np.ndarray) -> np.ndarray:
    """fp32 [N][K] -> Q6_K-style superblocks u8 [N][K/256*210]."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 256 == 0
    out = np.empty((N, K // 256 * 210), np.uint8)
    lib().moegen_quant_q6k(_p(W), N, K, _p(out))
    return out


def quant_q8_0(W: np.ndarray) -> np.ndarray:
    """fp32 [N][K] -> Q8_0-style blocks u8 [N][K/32*34]."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 32 == 0
    out = np.empty((N, K // 32 * 34), np.uint8)
    lib().moegen_quant_q8_0(_p(W), N, K, _p(out))
    return out


def quant_iq3g(W: np.ndarray) -> np.ndarray:
    """fp32 [N][K] -> IQ3-style grid rows [N][K/256*102] (see moegen.c)."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 256 == 0
    out = np.empty((N, K // 256 * 102), np.uint8)
    lib().moegen_quant_iq3g(_p(W), N, K, _p(out))
    return out


def quant_iq1g(W: np.ndarray) -> np.ndarray:
    """fp32 [N][K] -> IQ1-style ternary-grid rows [N][K/256*46] (see moegen.c)."""
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    assert K % 256 == 0
    out = np.empty((N, K // 256 * 46), np.uint8)
    lib().moegen_quant_iq1g(_p(W), N, K, _p(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().moegen_permutation(k, n, _p(out))
    return out


def zipf_bias(k: int, E: int, s: float, alpha: float):
    bias = np.empty(E, np.float32)
    rank = np.empty(E, np.int32)
    lib().moegen_zipf_bias(k, E, s, alpha, _p(bias), _p(rank))
    return bias, rank


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    E: int
    k: int
    H: int
    I: int
    T: int                      # tokens of the timed / checked batch
    fmt_down: int = FMT_NVFP4
    x_std: float = 1.0
    w_std: float = 0.02         # router and expert weights ~N(0, w_std)
    zipf_s: float = 0.0         # 0: no router bias
    zipf_alpha: float = 0.0
    renormalize: int = 1
    seed: int = 0
    extra: dict = field(default_factory=dict)


# Zipf-bias strengths fitted with the oracle router; written by
# moegen/fit_zipf_alpha.py into zipf_alpha.json.
import json as _json

with open(os.path.join(_HERE, "zipf_alpha.json")) as _f:
    ZIPF_ALPHA = _json.load(_f)

WORKLOADS = {
    # 8 experts, top-2, hidden 256, intermediate 128, 4 tokens, NVFP4 everywhere
    "tiny": Workload("tiny", E=8, k=2, H=256, I=128, T=4),
    # 128 experts, top-8, hidden 2048, intermediate 768, decode batch 1..8
    "decode": Workload("decode", E=128, k=8, H=2048, I=768, T=8),
    # same layer, 16384 tokens, router biased toward a Zipf(1.1) load
    "prefill": Workload("prefill", E=128, k=8, H=2048, I=768, T=16384, zipf_s=1.1,
                        zipf_alpha=ZIPF_ALPHA["prefill"]),
    # 256 experts, top-8, hidden 2048, intermediate 512; down in Q6_K-style
    "mixed": Workload("mixed", E=256, k=8, H=2048, I=512, T=8, fmt_down=FMT_Q6K,
                      extra={"prefill_T": 4096}),
    # the decode layer with its down projection in Q8_0 (8-bit blocks of 32)
    "q8": Workload("q8", E=128, k=8, H=2048, I=768, T=8, fmt_down=FMT_Q8_0,
                   extra={"prefill_T": 4096}),
    # the decode layer with its down projection in the IQ3-style grid format
    "iq3": Workload("iq3", E=128, k=8, H=2048, I=768, T=8, fmt_down=FMT_IQ3G,
                    extra={"prefill_T": 4096}),
    # the decode layer with its down projection in the IQ1-style ternary grid
    "iq1": Workload("iq1", E=128, k=8, H=2048, I=768, T=8, fmt_down=FMT_IQ1G,
                    extra={"prefill_T": 4096}),
    # 48 stacked mixed layers with 96 of 256 experts resident per layer
    "tiered": Workload("tiered", E=256, k=8, H=2048, I=512, T=8, fmt_down=FMT_Q6K,
                       zipf_s=1.2, zipf_alpha=ZIPF_ALPHA["tiered"],
                       extra={"layers": 48, "resident": 96, "steps": 2048, "drift": 256}),
}


@dataclass
class LayerWeights:
    E: int
    k: int
    H: int
    I: int
    fmt_down: int
    w_router: np.ndarray            # f32 [E][H]
    bias: np.ndarray | None         # f32 [E]
    gate_q: np.ndarray              # u8 [E][I][H/2]
    gate_s: np.ndarray              # u8 [E][I][H/16]
    gate_ts: np.ndarray             # f32 [E]
    up_q: np.ndarray
    up_s: np.ndarray
    up_ts: np.ndarray
    down_q: np.ndarray              # NVFP4 u8 [E][H][I/2], Q6K u8 [E][H][I/256*210], Q8_0 u8 [E][H][I/32*34],
                                    # IQ3G u8 [E][H][I/256*102], IQ1G u8 [E][H][I/256*46]
    down_s: np.ndarray | None       # NVFP4 u8 [E][H][I/16]
    down_ts: np.ndarray | None      # NVFP4 f32 [E]
    renormalize: int = 1


def make_layer(w: Workload, layer: int = 0, seed: int | None = None) -> LayerWeights:
    """Router and expert weights of one layer of workload ``w``."""
    seed = w.seed if seed is None else seed
    E, H, I = w.E, w.H, w.I
    L = lib()
    wr = normal_f32(key(seed, TAG_ROUTER, layer), E * H, w.w_std).reshape(E, H)
    bias = None
    if w.zipf_s > 0:
        bias, _ = zipf_bias(key(seed, TAG_BIAS, layer, 0), E, w.zipf_s, w.zipf_alpha)
    scratch = np.empty(max(I * H, 1), np.float32)
    gq = np.empty((E, I, H // 2), np.uint8)
    gs = np.empty((E, I, H // 16), np.uint8)
    gts = np.empty(E, np.float32)
    uq = np.empty_like(gq)
    us = np.empty_like(gs)
    uts = np.empty(E, np.float32)
    if w.fmt_down == FMT_NVFP4:
        dq = np.empty((E, H, I // 2), np.uint8)
        ds = np.empty((E, H, I // 16), np.uint8)
        dts = np.empty(E, np.float32)
    elif w.fmt_down == FMT_Q8_0:
        dq = np.empty((E, H, I // 32 * 34), np.uint8)
        ds = None
        dts = None
    elif w.fmt_down == FMT_IQ3G:
        dq = np.empty((E, H, I // 256 * 102), np.uint8)
        ds = None
        dts = None
    elif w.fmt_down == FMT_IQ1G:
        dq = np.empty((E, H, I // 256 * 46), np.uint8)
        ds = None
        dts = None
    else:
        dq = np.empty((E, H, I // 256 * 210), np.uint8)
        ds = None
        dts = None
    ts = np.zeros(1, np.float32)
    for e in range(E):
        L.moegen_nvfp4_normal(key(seed, (TAG_GATE << 20) | e, layer), I, H, w.w_std,
                              _p(scratch), _p(gq[e]), _p(gs[e]), _p(ts))
        gts[e] = ts[0]
        L.moegen_nvfp4_normal(key(seed, (TAG_UP << 20) | e, layer), I, H, w.w_std,
                              _p(scratch), _p(uq[e]), _p(us[e]), _p(ts))
        uts[e] = ts[0]
        if w.fmt_down == FMT_NVFP4:
            L.moegen_nvfp4_normal(key(seed, (TAG_DOWN << 20) | e, layer), H, I, w.w_std,
                                  _p(scratch), _p(dq[e]), _p(ds[e]), _p(ts))
            dts[e] = ts[0]
        elif w.fmt_down == FMT_Q8_0:
            L.moegen_q8_0_normal(key(seed, (TAG_DOWN << 20) | e, layer), H, I, w.w_std,
                                 _p(scratch), _p(dq[e]))
        elif w.fmt_down == FMT_IQ3G:
            L.moegen_iq3g_normal(key(seed, (TAG_DOWN << 20) | e, layer), H, I, w.w_std,
                                 _p(scratch), _p(dq[e]))
        elif w.fmt_down == FMT_IQ1G:
            L.moegen_iq1g_normal(key(seed, (TAG_DOWN << 20) | e, layer), H, I, w.w_std,
                                 _p(scratch), _p(dq[e]))
        else:
            L.moegen_q6k_normal(key(seed, (TAG_DOWN << 20) | e, layer), H, I, w.w_std,
                                _p(scratch), _p(dq[e]))
    return LayerWeights(E, w.k, H, I, w.fmt_down, wr, bias, gq, gs, gts, uq, us, uts,
                        dq, ds, dts, w.renormalize)


def make_tokens(w: Workload, T: int, step: int = 0, layer: int = 0,
                seed: int | None = None) -> np.ndarray:
    """bf16 activations [T][H] ~ N(0, x_std) for one step."""
    seed = w.seed if seed is None else seed
    return normal_bf16(key(seed, TAG_X, layer, step), T * w.H, w.x_std).reshape(T, w.H)


def make_residual(w: Workload, T: int, step: int = 0, layer: int = 0,
                  seed: int | None = None) -> np.ndarray:
    seed = w.seed if seed is None else seed
    return normal_bf16(key(seed, TAG_RESID, layer, step), T * w.H, w.x_std).reshape(T, w.H)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)
