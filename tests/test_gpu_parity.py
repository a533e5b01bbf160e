"""GPU parity: every step of the HIP path against the oracle, element by
element, on the same seeded inputs.  Routing logits, indices, bucket arrays and
the histogram must match bit for bit; gate weights within 1e-6; the bf16 layer
output within max-abs 2e-2 and relative L2 5e-3, and the expert outputs y
within relative L2 5e-3 (h is rounded to bf16 before the down projection)."""
import numpy as np
import pytest

import moegen
import oracle
from parity_util import (Y_REL, check_block_edges, check_buckets, check_layer, check_route, rel_l2,
                         run_gpu)

pytestmark = pytest.mark.gpu

_layers = {}


def layer(name, **over):
    key = (name, tuple(sorted(over.items())))
    if key not in _layers:
        base = moegen.WORKLOADS[name] if name in moegen.WORKLOADS else None
        w = moegen.Workload(**{**base.__dict__, **over}) if base else moegen.Workload(name=name, **over)
        _layers[key] = (w, moegen.make_layer(w))
    return _layers[key]


def test_tiny_layer_full_parity():
    w, L = layer("tiny")
    x = moegen.make_tokens(w, w.T)
    res = moegen.make_residual(w, w.T)
    print("tiny", w)
    check_layer(L, x)
    check_layer(L, x, residual=res)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_decode_layer_parity(B):
    """Decode batches of 1-8 tokens and verification-sized batches of 16 and
    32 (a few slots with draft tokens): dequant-fused GEMV path, fused gating
    (T * k <= 256)."""
    w, L = layer("decode")
    x = moegen.make_tokens(w, B, step=B)
    print("decode B", B)
    check_layer(L, x)


@pytest.mark.parametrize("B", [1, 2, 4])
def test_decode_gate_up_in_24_row_slices(B):
    """Small decode batches whose 32-row gate/up grid would give the CUs at
    most 1.5 workgroups each run gate/up in 24-row slices when I is a multiple
    of 96: here I = 384 (16 slices of 24 rows), H = 1024 (4 granules per
    lane), 48 experts, top-6, with a residual.  The decode layer (I = 768) at
    batches 1 and 2 takes the same path in test_decode_layer_parity."""
    import torch
    import quantized_expert_ffn_router_amd as q
    w, L = layer("rows24", E=48, k=6, H=1024, I=384, T=B)
    x = moegen.make_tokens(w, B, step=B)
    print("rows24 B", B, flush=True)
    check_layer(L, x, residual=moegen.make_residual(w, B))
    # the gate/up kernel that also gates (moe_route_ffn) and the plain one
    # (moe_expert_ffn after moe_route and moe_bucket) give the same y
    dl = q.DeviceLayer(L)
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    ys = []
    for fused in (True, False):
        buf = q.StepBuffers(dl, B, 0)
        q.layer_forward(dl, buf, xd, B, None, fused_gating=fused)
        torch.cuda.synchronize()
        ys.append(buf.y[:B * L.k].float().cpu().numpy())
    assert np.array_equal(ys[0], ys[1])


def test_ragged_mid_layer_parity():
    # 37 tokens (ragged), 3 K-groups of 128 in the down projection over 2 waves
    w, L = layer("mid", E=32, k=4, H=512, I=384, T=37)
    x = moegen.make_tokens(w, w.T)
    check_layer(L, x, residual=moegen.make_residual(w, w.T))


def test_many_tokens_per_expert_and_multiblock_bucket():
    # 600 x 8 = 4800 assignments: multi-block bucketing; ~75 tokens per expert
    # selects the grouped GEMM (bf16 h), hence the layer-level y tolerance.
    w, L = layer("many", E=64, k=8, H=256, I=128, T=600)
    x = moegen.make_tokens(w, w.T)
    check_layer(L, x, tokens=list(range(0, 600, 7)), y_rel=5e-3)


def test_mixed_q6k_decode_parity():
    w, L = layer("mixed")
    x = moegen.make_tokens(w, 8)
    check_layer(L, x)


def test_bf16_expert_outputs():
    w, L = layer("mid", E=32, k=4, H=512, I=384, T=37)
    x = moegen.make_tokens(w, w.T, step=3)
    check_layer(L, x, y_dtype=1, y_rel=5e-3)


def test_no_renormalisation_and_k_equals_E():
    w, L = layer("tiny", k=8, renormalize=0)
    L.renormalize = 0
    x = moegen.make_tokens(w, 5)
    check_layer(L, x)


@pytest.mark.parametrize("T", [5, 70])
def test_more_than_eight_experts_per_token(T):
    """k = 12: the combine takes a token's assignments in a group of 8 and a
    partial group of 4, with one-wavefront blocks (T <= 64) and 256-thread
    blocks (T > 64)."""
    w, L = layer("k12", E=32, k=12, H=256, I=128, T=T)
    x = moegen.make_tokens(w, T, step=4)
    res = moegen.make_residual(w, T)
    print("k12", T, flush=True)
    check_layer(L, x, residual=res)


# The grouped GEMM rounds h (and Q6_K weights) to bf16 before the MFMAs, so
# its fp32 expert outputs are compared at the layer tolerance (rel L2 5e-3).
GEMM_Y_REL = 5e-3


@pytest.mark.parametrize("fmt_down,mode", [(1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2), (4, 1),
                                           (4, 2)])
def test_largest_hidden_and_intermediate(fmt_down, mode):
    """H = I = 8192, the largest supported sizes, with each down format: the
    decode GEMVs split K over 4 (gate/up, 16 groups a wave) and 8 (down)
    waves; the grouped GEMM runs 64 K steps and 32 down column tiles.  The
    weights' std is halved against the 2048-wide layers (scaled like
    1/sqrt(fan-in)) so the outputs stay near unit scale, where the absolute
    bar of 2e-2 is above one bf16 ulp of the output."""
    w, L = layer("maxhi", E=2, k=2, H=8192, I=8192, T=3, fmt_down=fmt_down, w_std=0.01)
    x = moegen.make_tokens(w, w.T)
    print("maxhi", fmt_down, mode, flush=True)
    check_layer(L, x, ffn_mode=mode, y_rel=GEMM_Y_REL if mode == 2 else Y_REL)


@pytest.mark.parametrize("T,mode", [(5, 0), (70, 1), (70, 2)])
def test_most_experts_and_largest_top_k(T, mode):
    """E = 1024 and k = 64, the largest supported: the iterative top-k over
    1024 logits, 64 assignments per token in the combine (8 groups of 8) and,
    at 70 tokens, 4480 assignments over ~1000 active experts."""
    w, L = layer("maxe", E=1024, k=64, H=256, I=128, T=70)
    x = moegen.make_tokens(w, T, step=T)
    print("maxe", T, mode, flush=True)
    check_layer(L, x, residual=moegen.make_residual(w, T), ffn_mode=mode,
                y_rel=GEMM_Y_REL if mode == 2 else Y_REL)


def test_prefill_routing_full_size_and_sampled_outputs():
    """16384 tokens with the Zipf-biased router (grouped GEMM path): logits,
    indices and bucket arrays for every token; outputs on a sample of tokens
    (bf16 expert outputs, as the prefill path stores them)."""
    w, L = layer("prefill")
    x = moegen.make_tokens(w, w.T)
    sample = list(range(0, w.T, 512)) + [w.T - 1]
    g, _ = check_layer(L, x, tokens=sample, y_dtype=1, y_rel=GEMM_Y_REL)
    (r, worst), n = check_block_edges(g, L, x)
    print(f"prefill block edges: {n} rows, rel L2 {r:.2e}, worst row {worst:.2e}", flush=True)
    counts = g["buckets"]["counts"]
    assert counts.sum() == w.T * w.k and counts.min() > 0
    assert counts.max() > 4 * counts.min()   # biased load


def test_repeat_runs_are_bit_identical():
    w, L = layer("mid", E=32, k=4, H=512, I=384, T=37)
    x = moegen.make_tokens(w, w.T, step=9)
    a = run_gpu(L, x)
    b = run_gpu(L, x)
    for key in ("logits", "idx", "w", "y", "out"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


def test_equal_logits_tie_to_lower_index():
    """All-zero router weights: every logit equal, so experts 0..k-1, w = 1/k."""
    w, L = layer("tiny")
    L0 = moegen.LayerWeights(**{**L.__dict__, "w_router": np.zeros_like(L.w_router)})
    x = moegen.make_tokens(w, 4)
    g = run_gpu(L0, x)
    assert (g["idx"] == np.arange(w.k)).all()
    assert np.allclose(g["w"], 1.0 / w.k, atol=0)
    check_route(g, L0, x)
    check_buckets(g["buckets"], g["idx"], w.E)


def test_many_experts_iterative_topk_and_single_block_bucket():
    # E = 512 > 256 takes the iterative top-k; 100 x 4 = 400 assignments take
    # the one-workgroup bucket kernel.
    w, L = layer("wide", E=512, k=4, H=256, I=128, T=100)
    x = moegen.make_tokens(w, w.T)
    check_layer(L, x)


@pytest.mark.parametrize("mode", [1, 2])
def test_both_ffn_families_on_the_same_ragged_batch(mode):
    # 600 tokens x top-8 over 64 experts: ragged M tails in every expert;
    # mode 1 forces the GEMV kernels, mode 2 the MFMA grouped GEMM.
    w, L = layer("many", E=64, k=8, H=256, I=128, T=600)
    x = moegen.make_tokens(w, w.T, step=5)
    check_layer(L, x, tokens=list(range(0, 600, 5)), ffn_mode=mode, y_rel=GEMM_Y_REL)


def test_gemm_multiple_column_tiles_and_k_steps():
    # H = 512 (4 down column tiles of 128, 8 K steps of 64), I = 384 (6 gate/up
    # column tiles, 6 K steps); experts with 1..~90 rows.
    w, L = layer("gemm_mid", E=16, k=4, H=512, I=384, T=300)
    x = moegen.make_tokens(w, w.T)
    check_layer(L, x, residual=moegen.make_residual(w, w.T), tokens=list(range(0, 300, 3)),
                ffn_mode=2, y_rel=GEMM_Y_REL)


def test_mixed_prefill_q6k_down_sampled():
    """4096-token prefill of the 256-expert layer with the Q6_K-style down
    projection on the grouped GEMM path."""
    w, L = layer("mixed")
    x = moegen.make_tokens(w, 4096, step=1)
    g, _ = check_layer(L, x, tokens=list(range(0, 4096, 128)), y_dtype=1, y_rel=GEMM_Y_REL)
    (r, worst), n = check_block_edges(g, L, x)
    print(f"mixed prefill block edges: {n} rows, rel L2 {r:.2e}, worst row {worst:.2e}", flush=True)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_q8_0_decode_parity(B):
    """The decode layer with a Q8_0 down projection: dequant-fused GEMV."""
    w, L = layer("q8")
    x = moegen.make_tokens(w, B, step=B + 1)
    print("q8 decode B", B, flush=True)
    check_layer(L, x)


@pytest.mark.parametrize("mode", [1, 2])
def test_q8_0_both_ffn_families_ragged(mode):
    # 600 tokens x top-8 over 64 experts, I = 384 (3 groups of 128, 3 K steps
    # of the GEMM): GEMV (mode 1) and grouped GEMM (mode 2) against the oracle.
    w, L = layer("q8_many", E=64, k=8, H=256, I=384, T=600, fmt_down=moegen.FMT_Q8_0)
    x = moegen.make_tokens(w, w.T, step=6)
    res = moegen.make_residual(w, w.T)
    print("q8 ragged mode", mode, flush=True)
    check_layer(L, x, residual=res, tokens=list(range(0, 600, 5)), ffn_mode=mode,
                y_rel=GEMM_Y_REL)


def test_q8_0_prefill_sampled():
    """4096-token prefill of the Q8_0 layer on the grouped GEMM path."""
    w, L = layer("q8")
    x = moegen.make_tokens(w, 4096, step=2)
    print("q8 prefill", flush=True)
    g, _ = check_layer(L, x, tokens=list(range(0, 4096, 128)), y_dtype=1, y_rel=GEMM_Y_REL)
    (r, worst), n = check_block_edges(g, L, x)
    print(f"q8 prefill block edges: {n} rows, rel L2 {r:.2e}, worst row {worst:.2e}", flush=True)


@pytest.mark.parametrize("x_std,w_std,fmt_down", [
    (3e5, 0.02, 1),   # token rows beyond the fp16 range: per-row scaled fp16 copy
    (1e-3, 0.02, 1),  # small activations: h scaled by the token's row scale
    (1.0, 4.0, 1),    # |h| beyond fp16 even after scaling: bf16 recompute
    (1e-3, 0.02, 2),  # the same with the Q6_K-style down projection
    (1.0, 4.0, 2),
    (3e5, 0.02, 3),   # the same with Q8_0
    (1e-3, 0.02, 3),
    (1.0, 4.0, 3),
    (3e5, 0.02, 4),   # the same with IQ3G
    (1e-3, 0.02, 4),
    (1.0, 4.0, 4),
    (3e5, 0.02, 5),   # the same with IQ1G
    (1e-3, 0.02, 5),
    (1.0, 4.0, 5),
])
def test_gemm_activation_magnitudes(x_std, w_std, fmt_down):
    """The grouped GEMM multiplies fp16 operands; the token rows and h carry
    per-row power-of-two scales and an h overflow redoes the FFN with bf16 h.
    Results stay within the relative bars at any activation magnitude (the
    absolute bar of the other tests is for unit-scale activations)."""
    I = 384 if fmt_down in (1, 3) else 512  # Q6_K, IQ3G and IQ1G need I % 256 == 0
    w, L = layer("gemm_mag", E=16, k=4, H=512, I=I, T=300, x_std=x_std, w_std=w_std,
                 fmt_down=fmt_down)
    x = moegen.make_tokens(w, w.T)
    g = run_gpu(L, x, ffn_mode=2)
    logits, idx, wt = check_route(g, L, x)
    ob = check_buckets(g["buckets"], idx, L.E)
    toks = list(range(0, w.T, 3))
    o_out, o_y = oracle.ffn_combine(L, x, idx, wt, None, toks, want_y=True)
    rows = [t * L.k + j for t in toks for j in range(L.k)]
    gy = g["y"][ob["asg_pos"][rows]]
    assert rel_l2(gy, o_y[rows]) <= GEMM_Y_REL, rel_l2(gy, o_y[rows])
    got = moegen.bf16_to_f32(g["out"][toks])
    ref = moegen.bf16_to_f32(o_out[toks])
    assert rel_l2(got, ref) <= 5e-3, rel_l2(got, ref)


@pytest.mark.parametrize("B,keep_y", [(8, True), (1, False), (4, False), (8, False)])
def test_graph_replay_matches_eager(B, keep_y):
    """The bench times decode steps replayed from a HIP graph: each replay of
    a captured step equals the eager step bit for bit (output, indices, gate
    weights), with eager steps on other inputs and synchronizations between
    the replays; for the step through moe_route_ffn + moe_combine (keep_y) and
    through moe_layer_forward (gating inside gate/up at batch 1, down and
    combine in one kernel at batches 4 and 8)."""
    import torch
    import quantized_expert_ffn_router_amd as q
    w, L = layer("decode")
    dl = q.DeviceLayer(L)
    buf = q.StepBuffers(dl, B)
    xa = torch.from_numpy(moegen.make_tokens(w, B, step=11).view(np.int16).copy()).cuda()
    xb = torch.from_numpy(moegen.make_tokens(w, B, step=12).view(np.int16).copy()).cuda()
    s = torch.cuda.Stream()

    def snap():
        return (buf.out[:B].clone(), buf.idx[:B].clone(), buf.w[:B].clone())

    with torch.cuda.stream(s):
        q.layer_forward(dl, buf, xa, B, stream=s, hist_shifts=None, keep_y=keep_y)
    torch.cuda.synchronize()
    ref = snap()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q.layer_forward(dl, buf, xa, B, stream=s, hist_shifts=None, keep_y=keep_y)
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(s):
            q.layer_forward(dl, buf, xb, B, stream=s, hist_shifts=None, keep_y=keep_y)
        torch.cuda.synchronize()
        other = snap()
        assert not torch.equal(other[0], ref[0])  # the buffers now hold another step
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        got = snap()
        for a, b, name in zip(got, ref, ("out", "idx", "w")):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
    del g


def _scale_down_block_scales(L, exp2):
    """Copy of layer L whose Q6_K / Q8_0 / IQ3G / IQ1G down block scales d (fp16)
    are multiplied by 2^exp2 (rounded to fp16 where the result is subnormal;
    the oracle reads the same bytes)."""
    import dataclasses
    dq = L.down_q.copy()
    flat = dq.reshape(-1)
    bsz, off = {moegen.FMT_Q8_0: (34, 0), moegen.FMT_IQ3G: (102, 0),
                moegen.FMT_IQ1G: (46, 0)}.get(L.fmt_down, (210, 208))
    at = np.arange(flat.size // bsz) * bsz + off
    d = (flat[at].astype(np.uint16) | (flat[at + 1].astype(np.uint16) << 8)).view(np.float16)
    d2 = (d.astype(np.float64) * 2.0 ** exp2).astype(np.float16)
    assert np.isfinite(d2).all()
    bits = d2.view(np.uint16)
    flat[at] = (bits & 0xff).astype(np.uint8)
    flat[at + 1] = (bits >> 8).astype(np.uint8)
    return dataclasses.replace(L, down_q=dq)


@pytest.mark.parametrize("fmt_down,exp2", [(3, 18), (3, -10), (2, 16), (2, -8), (4, 16), (4, -10),
                                           (5, 20), (5, -10)])
def test_gemm_down_weights_at_any_scale(fmt_down, exp2):
    """The grouped GEMM's fp16 down weights carry a per-expert power of two
    fixed at pack time from the expert's largest block scale: Q8_0 weights
    up to 16K (beyond the plain fp16 product q * d * 16) and Q6_K d * sc up to
    ~100 (beyond d * sc * 2^10 in fp16), IQ3G superblock scales d near 20
    (weights up to ~5K), IQ1G superblock scales d near 2,000 (weights up to ~60K), and
    block scales pushed into fp16's subnormal range,
    all match the oracle at the relative bars."""
    I = 384 if fmt_down == 3 else 512
    w, L0 = layer("gemm_scale", E=16, k=4, H=512, I=I, T=300, fmt_down=fmt_down)
    L = _scale_down_block_scales(L0, exp2)
    x = moegen.make_tokens(w, w.T, step=13)
    print("down scale", fmt_down, exp2, flush=True)
    g = run_gpu(L, x, ffn_mode=2)
    logits, idx, wt = check_route(g, L, x)
    ob = check_buckets(g["buckets"], idx, L.E)
    toks = list(range(0, w.T, 3))
    o_out, o_y = oracle.ffn_combine(L, x, idx, wt, None, toks, want_y=True)
    rows = [t * L.k + j for t in toks for j in range(L.k)]
    gy = g["y"][ob["asg_pos"][rows]]
    assert np.isfinite(gy).all()
    assert rel_l2(gy, o_y[rows]) <= GEMM_Y_REL, rel_l2(gy, o_y[rows])
    got = moegen.bf16_to_f32(g["out"][toks])
    ref = moegen.bf16_to_f32(o_out[toks])
    assert rel_l2(got, ref) <= 5e-3, rel_l2(got, ref)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_iq3g_decode_parity(B):
    """The decode layer with the IQ3-style grid down projection (own grid):
    dequant-fused GEMV with the grid in LDS."""
    w, L = layer("iq3")
    x = moegen.make_tokens(w, B, step=B + 2)
    print("iq3g decode B", B, flush=True)
    check_layer(L, x)


@pytest.mark.parametrize("mode", [1, 2])
def test_iq3g_both_ffn_families_ragged(mode):
    # 600 tokens x top-8 over 64 experts, I = 512 (4 groups of 128, 2
    # superblocks, 4 K steps of the GEMM): GEMV (mode 1) and grouped GEMM
    # (mode 2) against the oracle.
    w, L = layer("iq3_many", E=64, k=8, H=256, I=512, T=600, fmt_down=moegen.FMT_IQ3G)
    x = moegen.make_tokens(w, w.T, step=7)
    res = moegen.make_residual(w, w.T)
    print("iq3g ragged mode", mode, flush=True)
    check_layer(L, x, residual=res, tokens=list(range(0, 600, 5)), ffn_mode=mode,
                y_rel=GEMM_Y_REL)


def test_iq3g_prefill_sampled():
    """4096-token prefill of the IQ3G layer on the grouped GEMM path, with
    the first and last row of every 128-row block."""
    w, L = layer("iq3")
    x = moegen.make_tokens(w, 4096, step=3)
    print("iq3g prefill", flush=True)
    g, _ = check_layer(L, x, tokens=list(range(0, 4096, 128)), y_dtype=1, y_rel=GEMM_Y_REL)
    (r, worst), n = check_block_edges(g, L, x)
    print(f"iq3g prefill block edges: {n} rows, rel L2 {r:.2e}, worst row {worst:.2e}", flush=True)


@pytest.mark.parametrize("B", [1, 8, 32])
def test_iq1g_decode_parity(B):
    """The decode layer with the IQ1-style ternary-grid down projection (own
    grid): dequant-fused GEMV with the grid in LDS as bf16 pairs."""
    w, L = layer("iq1")
    x = moegen.make_tokens(w, B, step=B + 4)
    print("iq1g decode B", B, flush=True)
    check_layer(L, x)


@pytest.mark.parametrize("mode", [1, 2])
def test_iq1g_both_ffn_families_ragged(mode):
    # 600 tokens x top-8 over 64 experts, I = 512 (4 groups of 128, 2
    # superblocks, 4 K steps of the GEMM): GEMV (mode 1) and grouped GEMM
    # (mode 2) against the oracle.
    w, L = layer("iq1_many", E=64, k=8, H=256, I=512, T=600, fmt_down=moegen.FMT_IQ1G)
    x = moegen.make_tokens(w, w.T, step=9)
    res = moegen.make_residual(w, w.T)
    print("iq1g ragged mode", mode, flush=True)
    check_layer(L, x, residual=res, tokens=list(range(0, 600, 5)), ffn_mode=mode,
                y_rel=GEMM_Y_REL)


def test_iq1g_prefill_sampled():
    """4096-token prefill of the IQ1G layer on the grouped GEMM path, with
    the first and last row of every 128-row block."""
    w, L = layer("iq1")
    x = moegen.make_tokens(w, 4096, step=5)
    print("iq1g prefill", flush=True)
    g, _ = check_layer(L, x, tokens=list(range(0, 4096, 128)), y_dtype=1, y_rel=GEMM_Y_REL)
    (r, worst), n = check_block_edges(g, L, x)
    print(f"iq1g prefill block edges: {n} rows, rel L2 {r:.2e}, worst row {worst:.2e}", flush=True)
