"""Shared helpers of the GPU parity tests: run the layer through the C ABI and
compare each step with the oracle on the same seeded inputs."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import moegen
import oracle

# FFN output tolerance of the layer against the oracle (bf16 outputs).
MAX_ABS = 2e-2
REL_L2 = 5e-3
# Gate-weight tolerance (fp32 on the GPU against fp64 -> fp32 in the oracle).
W_ABS = 1e-6


def run_gpu(L, x, residual=None, y_dtype=0, T_max=None, repeat=1, ffn_mode=0):
    import torch
    import quantized_expert_ffn_router_amd as q
    T = x.shape[0]
    dl = q.DeviceLayer(L, ffn_mode=ffn_mode)
    buf = q.StepBuffers(dl, T_max or max(T, 1), y_dtype)
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    rd = None if residual is None else torch.from_numpy(residual.view(np.int16).copy()).cuda()
    for _ in range(repeat):
        q.layer_forward(dl, buf, xd, T, rd)
    torch.cuda.synchronize()
    A = T * L.k
    res = dict(
        logits=buf.logits[:T].cpu().numpy(),
        idx=buf.idx[:T].cpu().numpy(),
        w=buf.w[:T].cpu().numpy(),
        buckets=buf.bucket_view(L.E, T, L.k),
        y=buf.y[:A].float().cpu().numpy(),
        out=buf.out[:T].cpu().numpy().view(np.uint16),
        hist=buf.hist.cpu().numpy().view(np.uint32),
    )
    return res


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def check_route(g, L, x):
    logits = oracle.router_logits(x, L.w_router, L.bias, 0)
    idx, w = oracle.topk(logits, L.k, L.renormalize)
    assert np.array_equal(g["logits"].view(np.uint32), logits.view(np.uint32)), \
        f"logits differ at {np.argwhere(g['logits'] != logits)[:5]}"
    assert np.array_equal(g["idx"], idx)
    assert np.max(np.abs(g["w"] - w)) <= W_ABS
    return logits, idx, w


def check_buckets(gb, idx, E):
    ob = oracle.bucket(idx, E)
    for key in ("counts", "offsets", "sorted_asg", "asg_pos", "active"):
        assert np.array_equal(gb[key], ob[key]), key
    assert gb["n_active"] == ob["n_active"]
    return ob


def check_out(g_out, o_out):
    got = moegen.bf16_to_f32(g_out).astype(np.float64)
    ref = moegen.bf16_to_f32(o_out).astype(np.float64)
    err = np.abs(got - ref)
    r = rel_l2(got, ref)
    assert err.max() <= MAX_ABS, err.max()
    assert r <= REL_L2, r
    return float(err.max()), r


# Expert outputs y: both FFN families round h to bf16 before the down
# projection (relative error <= 2^-9 per element, about 1.1e-3 relative L2 on
# y for incoherent errors); the bar is the layer's own 5e-3.
Y_REL = 5e-3


def check_layer(L, x, residual=None, y_dtype=0, tokens=None, y_rel=Y_REL, ffn_mode=0):
    """Full-layer parity; FFN compared on `tokens` (all when None)."""
    g = run_gpu(L, x, residual, y_dtype, ffn_mode=ffn_mode)
    logits, idx, w = check_route(g, L, x)
    ob = check_buckets(g["buckets"], idx, L.E)
    o_out, o_y = oracle.ffn_combine(L, x, idx, w, residual, tokens, want_y=True)
    toks = range(x.shape[0]) if tokens is None else tokens
    rows = [t * L.k + j for t in toks for j in range(L.k)]
    gy = g["y"][ob["asg_pos"][rows]]
    assert rel_l2(gy, o_y[rows]) <= y_rel, rel_l2(gy, o_y[rows])
    stats = check_out(g["out"][list(toks)], o_out[list(toks)])
    h = oracle.hist(ob["counts"], np.zeros(L.E, np.uint32), 5, 10)
    assert np.array_equal(g["hist"], h)
    return g, stats


def oracle_y(L, x, idx, asg=None):
    """Oracle expert outputs y[a] (float64 [n][H]) of assignments a = t*k + j
    (all of them when asg is None), grouped by expert and run on a thread pool
    (each expert's weights decoded once; oracle.expert_rows)."""
    k = idx.shape[1]
    asg = np.arange(idx.size) if asg is None else np.asarray(asg, np.int64)
    e_of = idx.reshape(-1)[asg]
    t_of = asg // k
    out = np.empty((asg.size, L.H), np.float64)
    groups = [(int(e), np.nonzero(e_of == e)[0]) for e in np.unique(e_of)]

    def run(g):
        e, rows = g
        out[rows] = oracle.expert_rows(L, e, x[t_of[rows]])

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(run, groups))
    return out


def block_edge_rows(counts, offsets, bm=128):
    """Sorted positions of the first and last row of every row block of bm
    rows of every expert (the grouped GEMM's row blocks; each expert's last
    block is the ragged one)."""
    rows = []
    for e in range(len(counts)):
        c, o = int(counts[e]), int(offsets[e])
        for b0 in range(0, c, bm):
            rows.append(o + b0)
            rows.append(o + min(b0 + bm, c) - 1)
    return np.unique(np.asarray(rows, np.int64))


# Per-row bar on expert outputs: the aggregate bar holds over many rows; a
# single row is allowed 4x (one wrong row still fails it).
Y_ROW_REL = 2e-2


def check_y_rows(gy, oy):
    """gy, oy: [n][H] expert outputs (GPU, oracle) of the same assignments."""
    gy = np.asarray(gy, np.float64)
    oy = np.asarray(oy, np.float64)
    r = rel_l2(gy, oy)
    assert r <= Y_REL, r
    num = np.linalg.norm(gy - oy, axis=1)
    den = np.maximum(np.linalg.norm(oy, axis=1), 1e-30)
    worst = int(np.argmax(num / den))
    assert (num / den).max() <= Y_ROW_REL, (worst, float((num / den).max()))
    return r, float((num / den).max())


def check_block_edges(g, L, x):
    """Expert outputs of the first and last row of every 128-row block of
    every expert (so each expert's ragged last block) against the oracle."""
    gb = g["buckets"]
    rows = block_edge_rows(gb["counts"], gb["offsets"])
    asg = gb["sorted_asg"][rows]
    oy = oracle_y(L, x, g["idx"], asg)
    return check_y_rows(g["y"][rows], oy), rows.size
