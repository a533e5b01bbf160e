"""Plumbing for stacks of MoE layers (torch memory and streams only; every
step runs in libmoe).  Used by the tiered-expert tests and benchmark.

A stack has L layers; layer l has its own router weights and, per drift
epoch, its own router bias; its experts are expert set l % n_sets of the
given host weights (sets may be shared between layers).  Each layer's output
feeds the next through the combine's residual: x_{l+1} = bf16(x_l + moe_l(x_l)).
"""
from __future__ import annotations

import numpy as np

from . import (DeviceLayer, LayerDesc, MOE_FMT_NVFP4, StepBuffers, TierDesc, moe_combine,
               moe_expert_blob_bytes, moe_expert_ffn, moe_route_bucket, moe_tier_create,
               moe_tier_destroy, moe_tier_prepare, moe_tier_prepare_async, moe_tier_rebalance)


def _pin(nbytes, pinned=True):
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=pinned)


class LayerStack:
    """routers: list of (w_router f32 [E][H]) per layer; biases(l, epoch) ->
    f32 [E] or None; expert_sets: list of moegen.LayerWeights (experts used)."""

    def __init__(self, expert_sets, routers, biases, L, k, renormalize=1, tiered=None):
        import torch
        dev = torch.device("cuda")
        s0 = expert_sets[0]
        self.E, self.H, self.I, self.k, self.L = s0.E, s0.H, s0.I, k, L
        self.fmt_down = s0.fmt_down
        self.renorm = renormalize
        self.eb = moe_expert_blob_bytes(self.H, self.I, MOE_FMT_NVFP4, self.fmt_down)
        self.n_sets = len(expert_sets)
        self.routers = [torch.from_numpy(np.ascontiguousarray(r)).to(dev) for r in routers]
        self.bias_fn = biases
        self._bias_cache = {}
        self.tiered = tiered
        # per-set expert scales (the table template)
        self.scales = []
        for w in expert_sets:
            refs = np.zeros(self.E, dtype=[("blob", "<u8"), ("tg", "<f4"), ("tu", "<f4"),
                                           ("td", "<f4"), ("r", "<u4")])
            refs["tg"] = w.gate_ts
            refs["tu"] = w.up_ts
            refs["td"] = w.down_ts if w.down_ts is not None else 1.0
            self.scales.append(refs)
        if tiered is None:
            # every expert resident: one DeviceLayer per set
            self.dev_sets = [DeviceLayer(w) for w in expert_sets]
            self.tables = [self.dev_sets[l % self.n_sets].refs for l in range(L)]
        else:
            R, S = tiered["resident"], tiered["staging"]
            # pack each set on the GPU, keep the blobs in pinned host memory
            self.host_sets = []
            for w in expert_sets:
                d = DeviceLayer(w)
                # pageable host blobs ("pinned": False) take the tier's
                # runtime-copy path instead of its copy kernel
                hb = _pin(self.E * self.eb, tiered.get("pinned", True))
                hb.copy_(d.blobs.cpu())
                self.host_sets.append(hb)
                del d
            torch.cuda.empty_cache()
            ptrs = np.zeros(L * self.E, np.uint64)
            scal = np.zeros(L * self.E, dtype=self.scales[0].dtype)
            for l in range(L):
                base = self.host_sets[l % self.n_sets].data_ptr()
                ptrs[l * self.E:(l + 1) * self.E] = base + np.arange(self.E, dtype=np.uint64) * self.eb
                scal[l * self.E:(l + 1) * self.E] = self.scales[l % self.n_sets]
            self._ptrs, self._scal = ptrs, scal
            self.pool_bytes = (L * R + S) * self.eb
            self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=dev)
            self.copy_stream = torch.cuda.Stream()
            desc = TierDesc(L, self.E, R, S, self.eb, ptrs.ctypes.data, scal.ctypes.data,
                            self.pool.data_ptr(), self.pool_bytes, self.copy_stream.cuda_stream)
            self.tier = moe_tier_create(desc)
            self.tables = [torch.zeros(self.E * 24, dtype=torch.uint8, device=dev) for _ in range(L)]
        self.descs = []
        for l in range(L):
            self.descs.append(LayerDesc(self.E, k, self.H, self.I, MOE_FMT_NVFP4, self.fmt_down,
                                        renormalize, 0, self.tables[l].data_ptr(),
                                        self.routers[l].data_ptr(), None))
        self.hists = [torch.zeros(self.E, dtype=torch.int32, device=dev) for _ in range(L)]
        self.buf = None

    def bias(self, l, epoch):
        key = (l, epoch)
        if key not in self._bias_cache:
            import torch
            b = self.bias_fn(l, epoch)
            self._bias_cache[key] = None if b is None else torch.from_numpy(b).cuda()
        return self._bias_cache[key]

    def close(self):
        if self.tiered is not None and getattr(self, "tier", None):
            moe_tier_destroy(self.tier)
            self.tier = None

    def step(self, x, T, epoch=0, stream=None, hist_shifts=(5, 10), trace=None):
        """One pass of all L layers over x (bf16 [T][H], updated in place).
        trace (list): receives a copy of each layer's input."""
        if self.buf is None or self.buf.T_max < T:
            # all layers share shape; buffers sized from layer 0's descriptor
            class _L:  # minimal stand-in with the fields StepBuffers reads
                pass
            d = _L()
            d.E, d.k, d.H, d.desc = self.E, self.k, self.H, self.descs[0]
            self.buf = StepBuffers(d, T)
        buf = self.buf
        for l in range(self.L):
            if trace is not None:
                trace.append(x.clone())
            desc = self.descs[l]
            b = self.bias(l, epoch)
            desc.router_bias = None if b is None else b.data_ptr()
            # route, top-k, bucketing and the usage histogram (one launch
            # after the router when the step is small enough)
            moe_route_bucket(desc, x, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                             buf.ws_bytes, self.hists[l], hist_shifts[0], hist_shifts[1], stream)
            if self.tiered is not None:
                prepare = moe_tier_prepare_async if self.tiered.get("async") else moe_tier_prepare
                prepare(self.tier, l, buf.buckets, self.tables[l], stream)
            moe_expert_ffn(desc, x, T, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes, stream)
            moe_combine(desc, buf.y, buf.y_dtype, buf.buckets, buf.w, T, x, x, stream)
        return x

    def rebalance(self, stream=None):
        for l in range(self.L):
            moe_tier_rebalance(self.tier, l, self.hists[l], stream)
