"""Cold-expert tier on the GPU: a stack of layers whose non-resident experts
are copied from pinned host memory on demand must compute bit-for-bit what
the same stack computes with every expert resident; residency follows the
usage histogram; a tiered layer matches the oracle (teacher-forced)."""
import numpy as np
import pytest

import moegen
import oracle
from parity_util import check_out

pytestmark = pytest.mark.gpu


def _stack_inputs(L=3, n_sets=2, E=64, k=4, H=256, I=256, s=1.2, alpha=0.39):
    w = moegen.Workload("tierstack", E=E, k=k, H=H, I=I, T=8, fmt_down=moegen.FMT_Q6K)
    sets = [moegen.make_layer(w, layer=i) for i in range(n_sets)]
    routers = [moegen.normal_f32(moegen.key(0, moegen.TAG_ROUTER, 1000 + l), E * H, 0.02)
               .reshape(E, H) for l in range(L)]

    def bias(l, epoch):
        b, _ = moegen.zipf_bias(moegen.key(0, moegen.TAG_BIAS, l, epoch), E, s, alpha)
        return b
    return w, sets, routers, bias


def _run(stack, w, steps, rebalance_every=None):
    import torch
    outs = []
    for st in range(steps):
        x = torch.from_numpy(moegen.make_tokens(w, 8, step=st).view(np.int16).copy()).cuda()
        stack.step(x, 8, epoch=st // 2)
        if rebalance_every and (st + 1) % rebalance_every == 0:
            stack.rebalance()
        torch.cuda.synchronize()
        outs.append(x.cpu().numpy().copy())
    return outs


def test_tiered_stack_equals_all_resident_bit_exact():
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs()
    ref = LayerStack(sets, routers, bias, L=3, k=w.k)
    tiered = LayerStack(sets, routers, bias, L=3, k=w.k,
                        tiered={"resident": 16, "staging": 32})
    a = _run(ref, w, 6)
    b = _run(tiered, w, 6, rebalance_every=2)
    for st, (u, v) in enumerate(zip(a, b)):
        assert np.array_equal(u, v), f"step {st} differs"
    import quantized_expert_ffn_router_amd as q
    stats, _ = q.moe_tier_stats_get(tiered.tier)
    assert stats["prepares"] == 6 * 3 and stats["rebalances"] == 3 * 3
    assert stats["hits"] > 0 and stats["misses"] > 0
    assert stats["h2d_bytes"] == (stats["misses"] + stats["promotions"]) * tiered.eb
    tiered.close()


def test_runtime_copy_path_equals_all_resident_bit_exact():
    """Host blobs in pageable memory are not mapped for the device, so the
    tier copies with one runtime copy per expert instead of its copy kernel;
    the results are the same bits."""
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs(L=2)
    ref = LayerStack(sets, routers, bias, L=2, k=w.k)
    tiered = LayerStack(sets, routers, bias, L=2, k=w.k,
                        tiered={"resident": 16, "staging": 32, "pinned": False})
    a = _run(ref, w, 4)
    b = _run(tiered, w, 4, rebalance_every=2)
    for st, (u, v) in enumerate(zip(a, b)):
        assert np.array_equal(u, v), f"step {st} differs"
    import quantized_expert_ffn_router_amd as q
    stats, _ = q.moe_tier_stats_get(tiered.tier)
    assert stats["misses"] > 0 and stats["promotions"] > 0
    tiered.close()


def test_rebalance_keeps_top_R_by_histogram():
    import torch
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs(L=2)
    st = LayerStack(sets, routers, bias, L=2, k=w.k, tiered={"resident": 16, "staging": 32})
    rng = np.random.default_rng(3)
    h = rng.integers(0, 50, size=w.E).astype(np.int32)  # many ties
    st.hists[1].copy_(torch.from_numpy(h))
    st.rebalance()
    torch.cuda.synchronize()
    _, res = q.moe_tier_stats_get(st.tier, layer=1, R=16)
    order = sorted(range(w.E), key=lambda e: (-int(h[e]), e))[:16]
    assert sorted(res.tolist()) == sorted(order)
    st.close()


def test_staging_overflow_is_reported():
    import torch
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs(L=1)
    st = LayerStack(sets, routers, bias, L=1, k=w.k, tiered={"resident": 0, "staging": 2})
    x = torch.from_numpy(moegen.make_tokens(w, 8).view(np.int16).copy()).cuda()
    with pytest.raises(q.MoeError) as ei:
        st.step(x, 8)
    assert ei.value.status == q.MOE_ERR_BUDGET
    torch.cuda.synchronize()
    st.close()


def test_tiered_layers_match_oracle_teacher_forced():
    import torch
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs(L=3)
    st = LayerStack(sets, routers, bias, L=3, k=w.k, tiered={"resident": 8, "staging": 32})
    x = torch.from_numpy(moegen.make_tokens(w, 8, step=7).view(np.int16).copy()).cuda()
    trace = []
    st.step(x, 8, epoch=1, trace=trace)
    torch.cuda.synchronize()
    ins = [t.cpu().numpy().view(np.uint16) for t in trace] + [x.cpu().numpy().view(np.uint16)]
    for l in range(3):
        Lw = sets[l % 2]
        layer = moegen.LayerWeights(**{**Lw.__dict__, "w_router": routers[l], "bias": bias(l, 1)})
        ref = oracle.layer(ins[l], layer, residual=ins[l])
        check_out(ins[l + 1], ref["out"])
    st.close()


def test_async_prepare_equals_sync_prepare_and_all_resident():
    """moe_tier_prepare_async (planning and copies on the device, no host
    round trip): the stack's outputs equal the all-resident stack's bit for
    bit, and hits, misses and copied bytes equal those of the synchronous
    prepare on the same steps."""
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs()
    ref = LayerStack(sets, routers, bias, L=3, k=w.k)
    sync = LayerStack(sets, routers, bias, L=3, k=w.k, tiered={"resident": 16, "staging": 32})
    asyn = LayerStack(sets, routers, bias, L=3, k=w.k,
                      tiered={"resident": 16, "staging": 32, "async": True})
    a = _run(ref, w, 6)
    b = _run(sync, w, 6, rebalance_every=2)
    c = _run(asyn, w, 6, rebalance_every=2)
    for st, (u, v) in enumerate(zip(a, c)):
        assert np.array_equal(u, v), f"step {st} differs"
    s_sync, _ = q.moe_tier_stats_get(sync.tier)
    s_async, _ = q.moe_tier_stats_get(asyn.tier)
    print("sync", s_sync, "async", s_async)
    for key in ("hits", "misses", "h2d_bytes", "promotions", "prepares", "rebalances"):
        assert s_async[key] == s_sync[key], key
    assert s_async["misses"] > 0 and s_async["hits"] > 0
    sync.close()
    asyn.close()


def test_async_prepare_needs_staging_for_every_possible_miss():
    """8 tokens x top-4 can miss 32 experts: 16 staging slots are refused
    before any launch; pageable host blobs are refused too (the device cannot
    read them)."""
    import torch
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs(L=1)
    x = torch.from_numpy(moegen.make_tokens(w, 8).view(np.int16).copy()).cuda()
    st = LayerStack(sets, routers, bias, L=1, k=w.k,
                    tiered={"resident": 8, "staging": 16, "async": True})
    with pytest.raises(q.MoeError) as ei:
        st.step(x, 8)
    assert ei.value.status == q.MOE_ERR_BUDGET
    torch.cuda.synchronize()
    st.close()
    st = LayerStack(sets, routers, bias, L=1, k=w.k,
                    tiered={"resident": 8, "staging": 32, "async": True, "pinned": False})
    with pytest.raises(q.MoeError) as ei:
        st.step(x, 8)
    assert ei.value.status == q.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    st.close()


def test_tiered_full_size_equals_all_resident_bit_exact():
    """The tiered configuration at full size, as the bench runs it: 48 layers
    of 256 experts (hidden 2048, intermediate 512, Q6_K-style down), 96
    resident per layer, 64 staging slots, the device-side prepare, a
    rebalance every 4 steps and Zipf(1.2) routing whose ranking is redrawn
    inside the run.  12 steps of 8 tokens equal the all-resident stack bit
    for bit (two expert sets shared round-robin by the layers); the first and
    last layers of the last step match the oracle (teacher-forced)."""
    import torch
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    W = moegen.WORKLOADS["tiered"]
    L, R, S, T = W.extra["layers"], W.extra["resident"], 64, W.T
    sets = [moegen.make_layer(W, layer=200 + i) for i in range(2)]
    routers = [moegen.normal_f32(moegen.key(0, moegen.TAG_ROUTER, 300 + l), W.E * W.H, W.w_std)
               .reshape(W.E, W.H) for l in range(L)]

    def bias(l, epoch):
        b, _ = moegen.zipf_bias(moegen.key(0, moegen.TAG_BIAS, 300 + l, epoch), W.E, W.zipf_s,
                                W.zipf_alpha)
        return b
    ref = LayerStack(sets, routers, bias, L=L, k=W.k)
    tiered = LayerStack(sets, routers, bias, L=L, k=W.k,
                        tiered={"resident": R, "staging": S, "async": True})
    steps, epoch_len = 12, 6
    trace = []
    for st in range(steps):
        x0 = moegen.make_tokens(W, T, step=st, layer=999).view(np.int16)
        xa = torch.from_numpy(x0.copy()).cuda()
        xb = torch.from_numpy(x0.copy()).cuda()
        ref.step(xa, T, epoch=st // epoch_len)
        tiered.step(xb, T, epoch=st // epoch_len, trace=trace if st == steps - 1 else None)
        if (st + 1) % 4 == 0:
            tiered.rebalance()
        torch.cuda.synchronize()
        assert torch.equal(xa, xb), f"step {st} differs"
    print("full-size tiered steps equal", flush=True)
    stats, _ = q.moe_tier_stats_get(tiered.tier)
    assert stats["hits"] > 0 and stats["misses"] > 0 and stats["promotions"] > 0
    ins = [t.cpu().numpy().view(np.uint16) for t in trace] + [xb.cpu().numpy().view(np.uint16)]
    ep = (steps - 1) // epoch_len
    for l in (0, L - 1):
        Lw = sets[l % 2]
        layer = moegen.LayerWeights(**{**Lw.__dict__, "w_router": routers[l], "bias": bias(l, ep)})
        out = oracle.layer(ins[l], layer, residual=ins[l])
        check_out(ins[l + 1], out["out"])
    tiered.close()
    ref.close()


def _permuted(w, perm):
    """Layer weights whose expert e is expert perm[e] of w (host arrays)."""
    d = dict(w.__dict__)
    for name in ("gate_q", "gate_s", "gate_ts", "up_q", "up_s", "up_ts", "down_q", "down_s",
                 "down_ts"):
        if d[name] is not None:
            d[name] = np.ascontiguousarray(d[name][perm])
    return moegen.LayerWeights(**d)


def test_per_layer_copies_with_permuted_experts():
    """layer_perms gives every layer its own copy of its set's blobs with the
    experts reordered: the tiered stack (per-layer pinned copies) equals the
    all-resident stack (per-layer device copies) bit for bit, and a layer
    matches the oracle run on the correspondingly permuted host weights."""
    import torch
    from quantized_expert_ffn_router_amd.stack import LayerStack
    L = 4
    w, sets, routers, bias = _stack_inputs(L=L)
    perms = [np.random.default_rng(50 + l).permutation(w.E) for l in range(L)]
    ref = LayerStack(sets, routers, bias, L=L, k=w.k, layer_perms=perms)
    tiered = LayerStack(sets, routers, bias, L=L, k=w.k, layer_perms=perms,
                        tiered={"resident": 16, "staging": 32, "async": True})
    assert tiered.host_bytes == L * w.E * tiered.eb
    trace = []
    for st in range(6):
        x0 = moegen.make_tokens(w, 8, step=st).view(np.int16)
        xa = torch.from_numpy(x0.copy()).cuda()
        xb = torch.from_numpy(x0.copy()).cuda()
        ref.step(xa, 8, epoch=st // 2, trace=trace if st == 5 else None)
        tiered.step(xb, 8, epoch=st // 2)
        if (st + 1) % 2 == 0:
            tiered.rebalance()
        torch.cuda.synchronize()
        assert torch.equal(xa, xb), f"step {st} differs"
    ins = [t.cpu().numpy().view(np.uint16) for t in trace] + [xa.cpu().numpy().view(np.uint16)]
    for l in (1, L - 1):
        Lw = _permuted(sets[l % len(sets)], perms[l])
        layer = moegen.LayerWeights(**{**Lw.__dict__, "w_router": routers[l], "bias": bias(l, 2)})
        out = oracle.layer(ins[l], layer, residual=ins[l])
        check_out(ins[l + 1], out["out"])
    tiered.close()
    ref.close()


def test_captured_tiered_step_equals_eager_all_resident():
    """The whole tiered step (route, bucket, device-side prepare, FFN and
    combine of every layer) captured once as a HIP graph and replayed 10
    times, with eager rebalances, epoch changes of the router bias and host
    synchronizations between the replays: every replay's output equals the
    eager all-resident step's bit for bit, and the tier's device counters
    advance as in eager steps."""
    import torch
    import quantized_expert_ffn_router_amd as q
    from quantized_expert_ffn_router_amd.stack import LayerStack
    w, sets, routers, bias = _stack_inputs()
    ref = LayerStack(sets, routers, bias, L=3, k=w.k)
    tiered = LayerStack(sets, routers, bias, L=3, k=w.k,
                        tiered={"resident": 16, "staging": 32, "async": True})
    tiered.use_bias_buffers(epoch=0)
    xg = torch.empty((8, w.H), dtype=torch.int16, device="cuda")
    g = tiered.capture(xg, 8)
    torch.cuda.synchronize()
    s0, _ = q.moe_tier_stats_get(tiered.tier)
    for st in range(10):
        x0 = moegen.make_tokens(w, 8, step=st).view(np.int16)
        xa = torch.from_numpy(x0.copy()).cuda()
        ref.step(xa, 8, epoch=st // 3)
        tiered.set_epoch(st // 3)
        xg.copy_(torch.from_numpy(x0.copy()))
        g.replay()
        if (st + 1) % 2 == 0:
            tiered.rebalance()
        torch.cuda.synchronize()
        assert torch.equal(xa, xg), f"replay {st} differs"
    s1, _ = q.moe_tier_stats_get(tiered.tier)
    assert s1["hits"] + s1["misses"] > s0["hits"] + s0["misses"]
    assert s1["misses"] > s0["misses"] and s1["promotions"] > 0
    del g
    tiered.close()
    ref.close()
