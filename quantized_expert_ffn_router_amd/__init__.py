"""Python binding of libmoe, the MI355X (gfx950) quantized mixture-of-experts layer.

This module only marshals arguments to the C ABI declared in ``include/moe.h``
(same entry-point names); every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and streams.  There is no fallback:
if ``libmoe.so`` is missing or fails to load, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_BUDGET = -4
MOE_ERR_HIP = -5
MOE_ERR_HOST_ALLOC = -6

MOE_FMT_NVFP4 = 1
MOE_FMT_Q6K = 2
MOE_FMT_Q8_0 = 3
MOE_FMT_IQ3G = 4
MOE_FMT_IQ1G = 5
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1

MOE_NOALLOC_WORKSPACE_BYTES = 32 << 20

MOE_FFN_AUTO = 0
MOE_FFN_GEMV = 1
MOE_FFN_GEMM = 2


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class ExpertRef(ctypes.Structure):
    _fields_ = [("blob", ctypes.c_void_p), ("ts_gate", ctypes.c_float),
                ("ts_up", ctypes.c_float), ("ts_down", ctypes.c_float),
                ("reserved", ctypes.c_uint32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("k", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32), ("fmt_gate_up", ctypes.c_int32),
                ("fmt_down", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("ffn_mode", ctypes.c_int32), ("experts", ctypes.c_void_p),
                ("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p)]


class Buckets(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sorted_asg", ctypes.c_void_p), ("asg_pos", ctypes.c_void_p),
                ("active", ctypes.c_void_p), ("n_active", ctypes.c_void_p),
                ("T_max", ctypes.c_int64), ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class TierDesc(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("E", ctypes.c_int32),
                ("resident_per_layer", ctypes.c_int32), ("staging_slots", ctypes.c_int32),
                ("expert_bytes", ctypes.c_size_t), ("host_blobs", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("hbm_pool", ctypes.c_void_p),
                ("hbm_pool_bytes", ctypes.c_size_t), ("copy_stream", ctypes.c_void_p)]


class TierStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("hits", "misses", "h2d_bytes", "promotions", "prepares", "rebalances")]


assert ctypes.sizeof(ExpertRef) == 24
assert ctypes.sizeof(TierDesc) == 64
assert ctypes.sizeof(LayerDesc) == 56
assert ctypes.sizeof(Buckets) == 64

# name -> (restype, argtypes); mirrors include/moe.h
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_LP = ctypes.POINTER(LayerDesc)
_BP = ctypes.POINTER(Buckets)
SIGNATURES = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_expert_blob_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "moe_pack_experts": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]),
    "moe_buckets_bytes": (_sz, [_i32, _i64, _i32]),
    "moe_buckets_carve": (ctypes.c_int, [_vp, _sz, _i32, _i64, _i32, _BP]),
    "moe_workspace_bytes": (_sz, [_LP, _i64]),
    "moe_route": (ctypes.c_int, [_LP, _vp, _i64, _vp, _vp, _vp, _vp]),
    "moe_bucket": (ctypes.c_int, [_LP, _vp, _i64, _BP, _vp, _sz, _vp]),
    "moe_expert_ffn": (ctypes.c_int, [_LP, _vp, _i64, _BP, _vp, _i32, _vp, _sz, _vp]),
    "moe_expert_ffn_noalloc": (ctypes.c_int, [_LP, _vp, _i64, _BP, _vp, _i32, _vp]),
    "moe_combine": (ctypes.c_int, [_LP, _vp, _i32, _BP, _vp, _i64, _vp, _vp, _vp]),
    "moe_expert_hist": (ctypes.c_int, [_LP, _BP, _vp, _i32, _i32, _vp]),
    "moe_route_ffn": (ctypes.c_int, [_LP, _vp, _i64, _vp, _vp, _vp, _BP, _vp, _i32, _i32, _vp,
                                      _i32, _vp, _sz, _vp]),
    "moe_layer_forward": (ctypes.c_int, [_LP, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _BP, _vp, _i32,
                                          _i32, _vp, _i32, _vp, _sz, _vp]),
    "moe_route_bucket": (ctypes.c_int, [_LP, _vp, _i64, _vp, _vp, _vp, _BP, _vp, _sz, _vp, _i32,
                                         _i32, _vp]),
    "moe_tier_create": (ctypes.c_int, [ctypes.POINTER(TierDesc), ctypes.POINTER(ctypes.c_void_p)]),
    "moe_tier_prepare": (ctypes.c_int, [_vp, _i32, _BP, _vp, _vp]),
    "moe_tier_prepare_async": (ctypes.c_int, [_vp, _i32, _BP, _vp, _vp]),
    "moe_tier_rebalance": (ctypes.c_int, [_vp, _i32, _vp, _vp]),
    "moe_tier_stats_get": (ctypes.c_int, [_vp, ctypes.POINTER(TierStats), _i32, _vp]),
    "moe_tier_destroy": (None, [_vp]),
}

_lib = None


def lib():
    """The loaded libmoe.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, last_error())


def _ptr(t) -> int | None:
    """Device (or host) address of a tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- raw ABI

def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_expert_blob_bytes(H, I, fmt_gate_up, fmt_down) -> int:
    return lib().moe_expert_blob_bytes(H, I, fmt_gate_up, fmt_down)


def moe_pack_experts(E, H, I, fmt_gate_up, fmt_down, gate_q, gate_s, up_q, up_s, down_q, down_s,
                     blobs, blob_stride, stream=None):
    _check(lib().moe_pack_experts(E, H, I, fmt_gate_up, fmt_down, _ptr(gate_q), _ptr(gate_s),
                                  _ptr(up_q), _ptr(up_s), _ptr(down_q), _ptr(down_s), _ptr(blobs),
                                  blob_stride, _stream(stream)))


def moe_buckets_bytes(E, T_max, k) -> int:
    return lib().moe_buckets_bytes(E, T_max, k)


def moe_buckets_carve(buf, nbytes, E, T_max, k) -> Buckets:
    b = Buckets()
    _check(lib().moe_buckets_carve(_ptr(buf), nbytes, E, T_max, k, ctypes.byref(b)))
    return b


def moe_workspace_bytes(desc: LayerDesc, T_max) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(desc), T_max)


def moe_route(desc, x, T, logits, topk_idx, topk_w, stream=None):
    _check(lib().moe_route(ctypes.byref(desc), _ptr(x), T, _ptr(logits), _ptr(topk_idx),
                           _ptr(topk_w), _stream(stream)))


def moe_bucket(desc, topk_idx, T, buckets, ws, ws_bytes, stream=None):
    _check(lib().moe_bucket(ctypes.byref(desc), _ptr(topk_idx), T, ctypes.byref(buckets),
                            _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn(desc, x, T, buckets, y, y_dtype, ws, ws_bytes, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(desc), _ptr(x), T, ctypes.byref(buckets), _ptr(y),
                                y_dtype, _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn_noalloc(desc, x, T, buckets, y, y_dtype, stream=None):
    _check(lib().moe_expert_ffn_noalloc(ctypes.byref(desc), _ptr(x), T, ctypes.byref(buckets),
                                        _ptr(y), y_dtype, _stream(stream)))


def moe_combine(desc, y, y_dtype, buckets, topk_w, T, residual, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(desc), _ptr(y), y_dtype, ctypes.byref(buckets),
                             _ptr(topk_w), T, _ptr(residual), _ptr(out), _stream(stream)))


def moe_expert_hist(desc, buckets, hist, decay_shift, unit_shift, stream=None):
    _check(lib().moe_expert_hist(ctypes.byref(desc), ctypes.byref(buckets), _ptr(hist),
                                 decay_shift, unit_shift, _stream(stream)))


def moe_route_bucket(desc, x, T, logits, topk_idx, topk_w, buckets, ws, ws_bytes, hist=None,
                     decay_shift=0, unit_shift=0, stream=None):
    _check(lib().moe_route_bucket(ctypes.byref(desc), _ptr(x), T, _ptr(logits), _ptr(topk_idx),
                                  _ptr(topk_w), ctypes.byref(buckets), _ptr(ws), ws_bytes,
                                  _ptr(hist), decay_shift, unit_shift, _stream(stream)))


def moe_route_ffn(desc, x, T, logits, topk_idx, topk_w, buckets, hist, decay_shift, unit_shift,
                  y, y_dtype, ws, ws_bytes, stream=None):
    _check(lib().moe_route_ffn(ctypes.byref(desc), _ptr(x), T, _ptr(logits), _ptr(topk_idx),
                               _ptr(topk_w), ctypes.byref(buckets), _ptr(hist), decay_shift,
                               unit_shift, _ptr(y), y_dtype, _ptr(ws), ws_bytes, _stream(stream)))


def moe_layer_forward(desc, x, T, residual, out, logits, topk_idx, topk_w, buckets, hist,
                      decay_shift, unit_shift, y, y_dtype, ws, ws_bytes, stream=None):
    _check(lib().moe_layer_forward(ctypes.byref(desc), _ptr(x), T, _ptr(residual), _ptr(out),
                                   _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                                   ctypes.byref(buckets), _ptr(hist), decay_shift, unit_shift,
                                   _ptr(y), y_dtype, _ptr(ws), ws_bytes, _stream(stream)))


def moe_tier_create(desc: TierDesc) -> int:
    h = ctypes.c_void_p()
    _check(lib().moe_tier_create(ctypes.byref(desc), ctypes.byref(h)))
    return h.value


def moe_tier_prepare(tier, layer, buckets, table_dev, stream=None):
    _check(lib().moe_tier_prepare(tier, layer, ctypes.byref(buckets), _ptr(table_dev),
                                  _stream(stream)))


def moe_tier_prepare_async(tier, layer, buckets, table_dev, stream=None):
    _check(lib().moe_tier_prepare_async(tier, layer, ctypes.byref(buckets), _ptr(table_dev),
                                        _stream(stream)))


def moe_tier_rebalance(tier, layer, hist, stream=None):
    _check(lib().moe_tier_rebalance(tier, layer, _ptr(hist), _stream(stream)))


def moe_tier_stats_get(tier, layer=0, R=0):
    st = TierStats()
    res = np.zeros(max(R, 1), np.int32)
    _check(lib().moe_tier_stats_get(tier, ctypes.byref(st), layer,
                                    res.ctypes.data if R else None))
    return {n: getattr(st, n) for n, _ in TierStats._fields_}, res[:R]


def moe_tier_destroy(tier):
    lib().moe_tier_destroy(tier)


# ---------------------------------------------------------------- device plumbing

class DeviceLayer:
    """One layer's weights resident in HBM: router weights/bias, packed expert
    blobs (packed on the GPU by moe_pack_experts) and the expert table.
    ffn_mode: MOE_FFN_AUTO, _GEMV or _GEMM, carried in the layer descriptor
    (desc.ffn_mode may be changed between calls)."""

    def __init__(self, w, device="cuda", stream=None, ffn_mode=MOE_FFN_AUTO):
        import torch
        self.E, self.k, self.H, self.I = w.E, w.k, w.H, w.I
        self.fmt_down = w.fmt_down
        dev = torch.device(device)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        self.w_router = t(w.w_router)
        self.bias = None if w.bias is None else t(w.bias)
        self.blob_bytes = moe_expert_blob_bytes(self.H, self.I, MOE_FMT_NVFP4, self.fmt_down)
        if self.blob_bytes == 0:
            raise MoeError(MOE_ERR_UNSUPPORTED, last_error())
        self.blobs = torch.empty(self.E * self.blob_bytes, dtype=torch.uint8, device=dev)
        canon = [t(a) if a is not None else None
                 for a in (w.gate_q, w.gate_s, w.up_q, w.up_s, w.down_q, w.down_s)]
        moe_pack_experts(self.E, self.H, self.I, MOE_FMT_NVFP4, self.fmt_down, *canon,
                         self.blobs, self.blob_bytes, stream)
        refs = np.zeros(self.E, dtype=[("blob", "<u8"), ("tg", "<f4"), ("tu", "<f4"),
                                       ("td", "<f4"), ("r", "<u4")])
        base = self.blobs.data_ptr()
        refs["blob"] = base + np.arange(self.E, dtype=np.uint64) * self.blob_bytes
        refs["tg"] = w.gate_ts
        refs["tu"] = w.up_ts
        refs["td"] = w.down_ts if w.down_ts is not None else 1.0
        self.refs = t(refs.view(np.uint8))
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        del canon
        self.desc = LayerDesc(self.E, self.k, self.H, self.I, MOE_FMT_NVFP4, self.fmt_down,
                              w.renormalize, ffn_mode, self.refs.data_ptr(), self.w_router.data_ptr(),
                              None if self.bias is None else self.bias.data_ptr())


class StepBuffers:
    """Per-step device buffers for up to T_max tokens of a layer."""

    def __init__(self, layer: DeviceLayer, T_max: int, y_dtype=MOE_DTYPE_F32, device="cuda"):
        import torch
        dev = torch.device(device)
        E, k, H = layer.E, layer.k, layer.H
        self.T_max = T_max
        self.y_dtype = y_dtype
        self.logits = torch.empty((T_max, E), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T_max, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T_max, k), dtype=torch.float32, device=dev)
        nb = moe_buckets_bytes(E, T_max, k)
        self.bucket_buf = torch.zeros(nb, dtype=torch.uint8, device=dev)
        self.buckets = moe_buckets_carve(self.bucket_buf, nb, E, T_max, k)
        self.ws_bytes = moe_workspace_bytes(layer.desc, T_max)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        ydt = torch.float32 if y_dtype == MOE_DTYPE_F32 else torch.bfloat16
        self.y = torch.empty((max(T_max * k, 1), H), dtype=ydt, device=dev)
        self.out = torch.empty((T_max, H), dtype=torch.int16, device=dev)
        self.hist = torch.zeros(E, dtype=torch.int32, device=dev)

    def counts_view(self, E: int):
        """The per-expert assignment counts of the last step as an int32
        device tensor view [E] (no copy)."""
        import torch
        off = self.buckets.counts - self.bucket_buf.data_ptr()
        return self.bucket_buf[off:off + 4 * E].view(torch.int32)

    def bucket_view(self, E: int, T: int, k: int) -> dict:
        """Host copies of the bucket outputs of the last step (synchronizes)."""
        b = self.bucket_buf.cpu().numpy()
        base = self.bucket_buf.data_ptr()

        def arr(ptr, n, dt):
            off = ptr - base
            return b[off: off + n * 4].view(dt).copy()
        bk = self.buckets
        A = T * k
        n_active = int(arr(bk.n_active, 1, np.int32)[0])
        return dict(counts=arr(bk.counts, E, np.uint32), offsets=arr(bk.offsets, E + 1, np.int32),
                    sorted_asg=arr(bk.sorted_asg, A, np.int32),
                    asg_pos=arr(bk.asg_pos, A, np.int32),
                    active=arr(bk.active, E, np.int32)[:n_active], n_active=n_active)


def layer_forward(layer: DeviceLayer, buf: StepBuffers, x, T: int, residual=None,
                  hist_shifts=(5, 10), stream=None, fused_gating=True, keep_y=True):
    """One pass of the layer: route, bucket, expert FFN, combine, histogram.
    fused_gating: one moe_route_ffn call (routing, gating, buckets, histogram
    and the expert FFN) in place of moe_route + moe_bucket + moe_expert_ffn +
    moe_expert_hist.  keep_y=False (with fused_gating): one moe_layer_forward
    call, which for decode batches fuses the down projection with the
    combine and leaves buf.y unwritten."""
    d = layer.desc
    if fused_gating and not keep_y:
        h = None if hist_shifts is None else buf.hist
        ds, us = (0, 0) if hist_shifts is None else hist_shifts
        moe_layer_forward(d, x, T, residual, buf.out, buf.logits, buf.idx, buf.w, buf.buckets, h,
                          ds, us, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes, stream)
        return buf.out
    if fused_gating:
        h = None if hist_shifts is None else buf.hist
        ds, us = (0, 0) if hist_shifts is None else hist_shifts
        moe_route_ffn(d, x, T, buf.logits, buf.idx, buf.w, buf.buckets, h, ds, us, buf.y,
                      buf.y_dtype, buf.ws, buf.ws_bytes, stream)
    else:
        moe_route(d, x, T, buf.logits, buf.idx, buf.w, stream)
        moe_bucket(d, buf.idx, T, buf.buckets, buf.ws, buf.ws_bytes, stream)
        moe_expert_ffn(d, x, T, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes, stream)
    moe_combine(d, buf.y, buf.y_dtype, buf.buckets, buf.w, T, residual, buf.out, stream)
    if hist_shifts is not None and not fused_gating:
        moe_expert_hist(d, buf.buckets, buf.hist, hist_shifts[0], hist_shifts[1], stream)
    return buf.out
