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
    f32 [E] or None; expert_sets: list of moegen.LayerWeights (experts used).

    layer_perms (optional, L int arrays of E): layer l's expert e is expert
    layer_perms[l][e] of its set, and every layer holds its own copy of its
    blobs (device memory when all-resident, pinned host memory when tiered),
    so the stack's footprint is that of L distinct layers."""

    def __init__(self, expert_sets, routers, biases, L, k, renormalize=1, tiered=None,
                 layer_perms=None):
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
        self.bias_bufs = None
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
        # each set packed once on the GPU
        packed = [DeviceLayer(w) for w in expert_sets]
        E, eb = self.E, self.eb

        def layer_scales(l):
            sc = self.scales[l % self.n_sets]
            return sc if layer_perms is None else sc[np.asarray(layer_perms[l])]

        def layer_blobs(l):  # device uint8 [E * eb]: layer l's experts in its order
            d = packed[l % self.n_sets].blobs
            if layer_perms is None:
                return d
            p = torch.from_numpy(np.asarray(layer_perms[l], dtype=np.int64)).to(dev)
            return d.view(E, eb)[p].reshape(-1)

        if tiered is None:
            if layer_perms is None:
                self.dev_sets = packed
                self.tables = [packed[l % self.n_sets].refs for l in range(L)]
            else:
                self.dev_blobs, self.tables = [], []
                for l in range(L):
                    blobs = layer_blobs(l)
                    refs = layer_scales(l).copy()
                    refs["blob"] = blobs.data_ptr() + np.arange(E, dtype=np.uint64) * eb
                    self.dev_blobs.append(blobs)
                    self.tables.append(torch.from_numpy(refs.view(np.uint8)).to(dev))
                del packed
        else:
            R, S = tiered["resident"], tiered["staging"]
            # blobs in host memory: pinned unless "pinned" is False (pageable
            # host blobs take the tier's runtime-copy path instead of its
            # copy kernel); one copy per set, or per layer with layer_perms
            n_host = self.n_sets if layer_perms is None else L
            self.host_sets = []
            for i in range(n_host):
                hb = _pin(E * eb, tiered.get("pinned", True))
                hb.copy_(layer_blobs(i) if layer_perms is not None else packed[i].blobs)
                self.host_sets.append(hb)
            del packed
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            ptrs = np.zeros(L * E, np.uint64)
            scal = np.zeros(L * E, dtype=self.scales[0].dtype)
            for l in range(L):
                base = self.host_sets[l if layer_perms is not None else l % self.n_sets].data_ptr()
                ptrs[l * E:(l + 1) * E] = base + np.arange(E, dtype=np.uint64) * eb
                scal[l * E:(l + 1) * E] = layer_scales(l)
            self._ptrs, self._scal = ptrs, scal
            self.host_bytes = n_host * E * eb
            self.pool_bytes = (L * R + S) * eb
            self.pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=dev)
            self.copy_stream = torch.cuda.Stream()
            desc = TierDesc(L, E, R, S, eb, ptrs.ctypes.data, scal.ctypes.data,
                            self.pool.data_ptr(), self.pool_bytes, self.copy_stream.cuda_stream)
            self.tier = moe_tier_create(desc)
            self.tables = [torch.zeros(E * 24, dtype=torch.uint8, device=dev) for _ in range(L)]
        self.descs = []
        for l in range(L):
            self.descs.append(LayerDesc(E, k, self.H, self.I, MOE_FMT_NVFP4, self.fmt_down,
                                        renormalize, 0, self.tables[l].data_ptr(),
                                        self.routers[l].data_ptr(), None))
        self.hists = [torch.zeros(E, dtype=torch.int32, device=dev) for _ in range(L)]
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

    def _buffers(self, T):
        if self.buf is None or self.buf.T_max < T:
            # all layers share shape; buffers sized from layer 0's descriptor
            class _L:  # minimal stand-in with the fields StepBuffers reads
                pass
            d = _L()
            d.E, d.k, d.H, d.desc = self.E, self.k, self.H, self.descs[0]
            self.buf = StepBuffers(d, T)
        return self.buf

    def use_bias_buffers(self, epoch=0):
        """From now on every layer reads its router bias from a fixed device
        buffer (epoch arguments of step are ignored; set_epoch refills the
        buffers), so that a captured step stays valid across epochs."""
        self.bias_bufs = None
        bufs = []
        for l in range(self.L):
            b = self.bias(l, epoch)
            bufs.append(None if b is None else b.clone())
        self.bias_bufs = bufs

    def set_epoch(self, epoch):
        """Copy epoch's router biases into the fixed buffers (torch's current
        stream)."""
        for l, buf in enumerate(self.bias_bufs):
            if buf is not None:
                buf.copy_(self.bias(l, epoch))

    def capture(self, x, T, hist_shifts=(5, 10)):
        """One step over x (bf16 [T][H], updated in place) recorded as a HIP
        graph: route, bucket, device-side tier prepare, FFN and combine of all
        L layers.  Needs use_bias_buffers and, when tiered, the device-side
        prepare (the host prepare waits on the host).  Replay on torch's
        current stream; rebalance between replays as between steps."""
        import torch
        if self.bias_bufs is None:
            raise ValueError("capture: call use_bias_buffers first")
        if self.tiered is not None and not self.tiered.get("async"):
            raise ValueError("capture: a tiered stack needs the device-side prepare")
        self._buffers(T)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=s):
            self.step(x, T, hist_shifts=hist_shifts)
        torch.cuda.current_stream().wait_stream(s)
        return g

    def step(self, x, T, epoch=0, stream=None, hist_shifts=(5, 10), trace=None, active_acc=None):
        """One pass of all L layers over x (bf16 [T][H], updated in place).
        trace (list): receives a copy of each layer's input.  active_acc
        (int32 [L][E] device tensor): 1 is added to entry [l][e] when expert e
        of layer l takes at least one token in this step (torch's current
        stream does the adds, so stream must be that stream or None)."""
        buf = self._buffers(T)
        for l in range(self.L):
            if trace is not None:
                trace.append(x.clone())
            desc = self.descs[l]
            b = self.bias(l, epoch) if self.bias_bufs is None else self.bias_bufs[l]
            desc.router_bias = None if b is None else b.data_ptr()
            # route, top-k, bucketing and the usage histogram (one launch
            # after the router when the step is small enough)
            moe_route_bucket(desc, x, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                             buf.ws_bytes, self.hists[l], hist_shifts[0], hist_shifts[1], stream)
            if active_acc is not None:
                active_acc[l] += buf.counts_view(self.E).gt(0)
            if self.tiered is not None:
                prepare = moe_tier_prepare_async if self.tiered.get("async") else moe_tier_prepare
                prepare(self.tier, l, buf.buckets, self.tables[l], stream)
            moe_expert_ffn(desc, x, T, buf.buckets, buf.y, buf.y_dtype, buf.ws, buf.ws_bytes, stream)
            moe_combine(desc, buf.y, buf.y_dtype, buf.buckets, buf.w, T, x, x, stream)
        return x

    def rebalance(self, stream=None):
        for l in range(self.L):
            moe_tier_rebalance(self.tier, l, self.hists[l], stream)
