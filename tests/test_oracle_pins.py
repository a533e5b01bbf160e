"""Pins of the CPU oracle against facts fixed outside it.

Each test ties one oracle function to something other than its own formula:
format tables of the OCP specifications (tests/golden), torch's float8 /
bfloat16 / numpy float16 decoders, exact rational arithmetic, brute-force
sorting, numpy's stable argsort, scipy's softmax and expit, and a dense fp64
reference of the whole layer on the tiny workload.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import moegen
import oracle
from conftest import load_golden


# ---------------------------------------------------------------- formats

def test_e2m1_matches_ocp_table():
    rows = load_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1(int(code))
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_matches_ocp_points_and_torch():
    for b, val in load_golden("e4m3_points.txt"):
        got = oracle.e4m3(int(b, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = oracle.e4m3(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), b
        else:
            assert got == ref[b], (b, got, ref[b])


def test_f16_bf16_decode_match_numpy_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, size=4000, dtype=np.uint16)
    f16 = bits.view(np.float16).astype(np.float64)
    bf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for i, b in enumerate(bits):
        g = oracle.f16(int(b))
        assert (math.isnan(g) and math.isnan(f16[i])) or g == f16[i]
        g = oracle.bf16(int(b))
        assert (math.isnan(g) and math.isnan(bf[i])) or g == bf[i]


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(2)
    vals = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                           [1.00390625, 1.005859375, -2.01171875, 3.0e-39, -1.0e-40]])
    vals = vals.astype(np.float32)  # exactly representable: one rounding in torch too
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(vals, ref):
        assert oracle.round_bf16(float(v)) == int(r), v


def test_nvfp4_decode_hand_built():
    e2m1 = {int(c): float(v) for c, v in load_golden("e2m1_values.txt")}
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rng = np.random.default_rng(3)
    N, K = 5, 64
    codes4 = rng.integers(0, 16, size=(N, K))
    scales = rng.integers(0, 127, size=(N, K // 16)).astype(np.uint8)
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    ts = np.float32(0.0123)
    got = oracle.decode_nvfp4(packed, scales, float(ts))
    for n in range(N):
        for k in range(K):
            exp = e2m1[int(codes4[n, k])] * e4m3[scales[n, k // 16]] * float(ts)
            assert got[n, k] == exp


def test_q6k_decode_closed_form():
    """Pack random integers by the documented byte layout; decode must equal
    d * sc * (q - 32) computed from the integers themselves."""
    rng = np.random.default_rng(4)
    N, K = 3, 512
    q = rng.integers(0, 64, size=(N, K))
    sc = rng.integers(-128, 128, size=(N, K // 16))
    d = (rng.standard_normal((N, K // 256)) * 1e-3).astype(np.float16)
    blocks = np.zeros((N, K // 256, 210), np.uint8)
    for n in range(N):
        for s in range(K // 256):
            for i in range(256):
                v = int(q[n, 256 * s + i])
                blocks[n, s, i // 2] |= (v & 15) << (4 * (i % 2))
                blocks[n, s, 128 + i // 4] |= ((v >> 4) & 3) << (2 * (i % 4))
            blocks[n, s, 192:208] = sc[n, 16 * s:16 * s + 16].astype(np.int8).view(np.uint8)
            blocks[n, s, 208:210] = np.frombuffer(d[n, s].tobytes(), np.uint8)
    got = oracle.decode_q6k(blocks.reshape(N, -1), K)
    for n in range(N):
        for k in range(K):
            exp = float(d[n, k // 256]) * float(sc[n, k // 16]) * float(q[n, k] - 32)
            assert got[n, k] == exp


def test_q8_0_decode_closed_form():
    """Pack random int8 codes and fp16 scales by the documented byte layout
    (d little-endian, then 32 codes per block); decode must equal d * q from
    the integers and numpy's float16 decoding of d."""
    rng = np.random.default_rng(6)
    N, K = 3, 256
    q = rng.integers(-128, 128, size=(N, K))
    d = (rng.standard_normal((N, K // 32)) * 1e-3).astype(np.float16)
    blocks = np.zeros((N, K // 32, 34), np.uint8)
    for n in range(N):
        for b in range(K // 32):
            blocks[n, b, 0:2] = np.frombuffer(d[n, b].tobytes(), np.uint8)
            blocks[n, b, 2:] = q[n, 32 * b:32 * b + 32].astype(np.int8).view(np.uint8)
    got = oracle.decode_q8_0(blocks.reshape(N, -1), K)
    for n in range(N):
        for k in range(K):
            assert got[n, k] == float(d[n, k // 32]) * float(q[n, k])


def test_q8_0_generator_roundtrip_on_grid():
    """Blocks whose values are d * integers with |q| <= 127 and one |q| = 127
    (so amax / 127 = d, an exact fp16 power of two) survive quantize -> decode
    exactly."""
    rng = np.random.default_rng(7)
    N, K = 4, 128
    qi = rng.integers(-127, 128, size=(N, K))
    qi[:, ::32] = 127 * np.where(rng.integers(0, 2, size=(N, K // 32)) > 0, 1, -1)
    W = (qi * 2.0 ** -9).astype(np.float32)
    dec = oracle.decode_q8_0(moegen.quant_q8_0(W), K)
    np.testing.assert_array_equal(dec, W.astype(np.float64))


def test_q8_0_generator_zero_block_and_code_range():
    """An all-zero block gets d = 0 and zero codes (decodes to zeros); in
    random blocks every code stays in [-127, 127] and each decoded weight is
    within d/2 of the input, except where the clamp at 127 applies (the
    block maximum, when fp16 rounds d below amax/127)."""
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((3, 96)) * 0.05).astype(np.float32)
    W[1, 32:64] = 0.0
    q = moegen.quant_q8_0(W).reshape(3, 3, 34)
    codes = q[:, :, 2:].view(np.int8).astype(np.int64)
    assert codes.min() >= -127 and codes.max() <= 127
    assert (q[1, 1] == 0).all()
    dec = oracle.decode_q8_0(moegen.quant_q8_0(W), 96)
    assert (dec[1, 32:64] == 0).all()
    d = q[:, :, :2].copy().view(np.float16).astype(np.float64)[:, :, 0]
    err = np.abs(dec - W.astype(np.float64)).reshape(3, 3, 32)
    clamped = (np.abs(codes) == 127)
    assert (err[~clamped] <= (d[:, :, None] / 2 + 1e-12).repeat(32, 2)[~clamped]).all()


def test_generator_quantizers_roundtrip_on_grid():
    """Values already on the NVFP4 / Q6_K grids survive quantize->decode."""
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    rng = np.random.default_rng(5)
    N, K = 4, 64
    W = rng.choice(np.concatenate([e2m1, -e2m1]), size=(N, K))
    W[:, 0] = 6.0  # each 16-block then has amax 6 in some rows; force exact scale
    for b in range(K // 16):
        W[:, 16 * b] = 6.0
    W = (W * 0.25).astype(np.float32)  # amax 1.5 -> ts = 1.5/2688
    codes, scales, ts = moegen.quant_nvfp4(W)
    dec = oracle.decode_nvfp4(codes, scales, ts)
    np.testing.assert_allclose(dec, W, rtol=2e-7, atol=0)


# ---------------------------------------------------------------- router

def _f32_rne_of_fraction(fr: Fraction) -> np.float32:
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr),
                                     int(np.array(c).view(np.uint32)) & 1))
    return best


def test_router_logits_equal_exact_rounding_tiny():
    W = moegen.WORKLOADS["tiny"]
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    bias = np.linspace(-0.3, 0.2, W.E).astype(np.float32)
    for order in (0, 1):
        got = oracle.router_logits(x, L.w_router, bias, order)
        xf = moegen.bf16_to_f32(x)
        for t in range(W.T):
            for e in range(W.E):
                s = sum(Fraction(float(a)) * Fraction(float(b))
                        for a, b in zip(xf[t], L.w_router[e]))
                s += Fraction(float(bias[e]))
                assert got[t, e] == _f32_rne_of_fraction(s), (order, t, e)


def test_router_orders_agree_at_decode_shape():
    W = moegen.WORKLOADS["decode"]
    rng_layer = moegen.make_layer(moegen.Workload("r", E=128, k=8, H=2048, I=128, T=8))
    x = moegen.make_tokens(W, 64)
    a = oracle.router_logits(x, rng_layer.w_router, None, 0)
    b = oracle.router_logits(x, rng_layer.w_router, None, 1)
    ref = (moegen.bf16_to_f32(x).astype(np.float64) @ rng_layer.w_router.T.astype(np.float64))
    assert np.array_equal(a, b)
    assert np.array_equal(a, ref.astype(np.float32))


# ---------------------------------------------------------------- top-k

def _brute_topk(l, k):
    order = sorted(range(len(l)), key=lambda e: (-float(l[e]), e))
    return order[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 8), (5, 5), (64, 1)])
def test_topk_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 200
    logits = (rng.integers(-6, 6, size=(T, E)) * 0.25).astype(np.float32)  # many ties
    idx, w = oracle.topk(logits, k, 1)
    for t in range(T):
        assert list(idx[t]) == _brute_topk(logits[t], k)
        ref = scipy.special.softmax(logits[t, idx[t]].astype(np.float64))
        np.testing.assert_allclose(w[t], ref, rtol=0, atol=1e-7)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 1e-6


def test_topk_special_cases():
    l = np.zeros((3, 16), np.float32)
    idx, w = oracle.topk(l, 4, 1)
    assert (idx == np.arange(4)).all() and np.allclose(w, 0.25, atol=0)
    rng = np.random.default_rng(7)
    l = rng.standard_normal((10, 16)).astype(np.float32)
    idx, w = oracle.topk(l, 1, 1)
    assert (w == 1.0).all() and (idx[:, 0] == np.argmax(l, axis=1)).all()
    idx, w = oracle.topk(l, 16, 1)
    for t in range(10):
        assert list(idx[t]) == _brute_topk(l[t], 16)
    idx, w = oracle.topk(l, 3, 0)  # no renormalisation: full softmax probabilities
    for t in range(10):
        p = scipy.special.softmax(l[t].astype(np.float64))
        np.testing.assert_allclose(w[t], p[idx[t]], rtol=0, atol=1e-7)


# ---------------------------------------------------------------- bucketing

@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (1, 8, 128), (300, 4, 32), (1000, 8, 256), (0, 8, 16)])
def test_bucket_matches_stable_argsort(T, k, E):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    b = oracle.bucket(idx, E)
    flat = idx.reshape(-1)
    assert (b["counts"] == np.bincount(flat, minlength=E)).all()
    assert b["offsets"][0] == 0 and (np.diff(b["offsets"]) == b["counts"]).all()
    assert (b["sorted_asg"] == np.argsort(flat, kind="stable")).all()
    assert (b["sorted_asg"][b["asg_pos"]] == np.arange(T * k)).all()
    assert (b["active"] == np.nonzero(b["counts"])[0]).all()


# ---------------------------------------------------------------- histogram

def test_hist_steps_and_fixed_point():
    h = oracle.hist(np.array([3, 0, 1], np.uint32), np.array([1000, 31, 0xFFFFFFFF], np.uint32), 5, 10)
    assert list(h) == [1000 - 31 + 3072, 31 - 0 + 0, (0xFFFFFFFF - (0xFFFFFFFF >> 5) + 1024) & 0xFFFFFFFF]
    s, u = 5, 10
    counts = np.array([0, 1, 2, 7, 8], np.uint32)
    hv = np.zeros(5, np.uint32)
    for _ in range(3000):
        hv = oracle.hist(counts, hv, s, u)
    for c, v in zip(counts, hv):
        C = int(c) << u
        assert C << s <= int(v) <= (C << s) + (1 << s) - 1   # v >> s == C
    assert (oracle.hist(counts, hv, s, u) == hv).all()


# ---------------------------------------------------------------- expert FFN

def _dense_reference(L, x, w_idx, w_val, residual=None):
    """Every token through every expert in fp64, combined with gate weights
    that are zero for unselected experts (no bucketing, no gather)."""
    e2m1 = np.array([float(v) for _, v in load_golden("e2m1_values.txt")])
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()

    def dq(codes, scales, ts):
        N, Kh = codes.shape
        c = np.empty((N, 2 * Kh), np.int64)
        c[:, 0::2] = codes & 15
        c[:, 1::2] = codes >> 4
        return e2m1[c] * np.repeat(e4m3[scales], 16, axis=1) * float(ts)

    xf = moegen.bf16_to_f32(x).astype(np.float64)
    T = x.shape[0]
    gates = np.zeros((T, L.E))
    for t in range(T):
        gates[t, w_idx[t]] = w_val[t]
    out = np.zeros((T, L.H))
    ys = {}
    for e in range(L.E):
        Wg = dq(L.gate_q[e], L.gate_s[e], L.gate_ts[e])
        Wu = dq(L.up_q[e], L.up_s[e], L.up_ts[e])
        if L.fmt_down == moegen.FMT_NVFP4:
            Wd = dq(L.down_q[e], L.down_s[e], L.down_ts[e])
        elif L.fmt_down == moegen.FMT_Q8_0:
            Wd = oracle.decode_q8_0(L.down_q[e], L.I)
        elif L.fmt_down == moegen.FMT_IQ3G:
            Wd = oracle.decode_iq3g(L.down_q[e], L.I)
        elif L.fmt_down == moegen.FMT_IQ1G:
            Wd = oracle.decode_iq1g(L.down_q[e], L.I)
        else:
            Wd = oracle.decode_q6k(L.down_q[e], L.I)
        g = xf @ Wg.T
        u = xf @ Wu.T
        h = g * scipy.special.expit(g) * u
        y = h @ Wd.T
        ys[e] = y
        out += gates[:, e:e + 1] * y
    if residual is not None:
        out += moegen.bf16_to_f32(residual).astype(np.float64)
    return out, ys


def _bf16_close(got_bits, ref, ulps=1):
    got = moegen.bf16_to_f32(got_bits).astype(np.float64)
    tol = ulps * np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
    assert (np.abs(got - ref) <= tol).all(), np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))


def test_ffn_tiny_dense_fp64_reference():
    W = moegen.WORKLOADS["tiny"]
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    res = moegen.make_residual(W, W.T)
    _, idx, w = oracle.route(x, L)
    out, y = oracle.ffn_combine(L, x, idx, w, residual=res, want_y=True)
    ref, ys = _dense_reference(L, x, idx, w, residual=res)
    for t in range(W.T):
        for j in range(W.k):
            np.testing.assert_allclose(y[t * W.k + j], ys[idx[t, j]][t], rtol=1e-12, atol=1e-15)
    _bf16_close(out, ref)


def test_ffn_q6k_down_dense_reference():
    W = moegen.Workload("q6", E=4, k=2, H=256, I=256, T=3, fmt_down=moegen.FMT_Q6K)
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    _, idx, w = oracle.route(x, L)
    out, y = oracle.ffn_combine(L, x, idx, w, want_y=True)
    ref, ys = _dense_reference(L, x, idx, w)
    for t in range(W.T):
        for j in range(W.k):
            np.testing.assert_allclose(y[t * W.k + j], ys[idx[t, j]][t], rtol=1e-12, atol=1e-15)
    _bf16_close(out, ref)


def test_ffn_q8_0_down_dense_reference():
    W = moegen.Workload("q8", E=4, k=2, H=256, I=256, T=3, fmt_down=moegen.FMT_Q8_0)
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    _, idx, w = oracle.route(x, L)
    out, y = oracle.ffn_combine(L, x, idx, w, want_y=True)
    ref, ys = _dense_reference(L, x, idx, w)
    for t in range(W.T):
        for j in range(W.k):
            np.testing.assert_allclose(y[t * W.k + j], ys[idx[t, j]][t], rtol=1e-12, atol=1e-15)
    _bf16_close(out, ref)


def test_ffn_iq3g_down_dense_reference():
    W = moegen.Workload("iq3", E=4, k=2, H=256, I=256, T=3, fmt_down=moegen.FMT_IQ3G)
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    _, idx, w = oracle.route(x, L)
    out, y = oracle.ffn_combine(L, x, idx, w, want_y=True)
    ref, ys = _dense_reference(L, x, idx, w)
    for t in range(W.T):
        for j in range(W.k):
            np.testing.assert_allclose(y[t * W.k + j], ys[idx[t, j]][t], rtol=1e-12, atol=1e-15)
    _bf16_close(out, ref)


def test_ffn_iq1g_down_dense_reference():
    W = moegen.Workload("iq1", E=4, k=2, H=256, I=256, T=3, fmt_down=moegen.FMT_IQ1G)
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    _, idx, w = oracle.route(x, L)
    out, y = oracle.ffn_combine(L, x, idx, w, want_y=True)
    ref, ys = _dense_reference(L, x, idx, w)
    for t in range(W.T):
        for j in range(W.k):
            np.testing.assert_allclose(y[t * W.k + j], ys[idx[t, j]][t], rtol=1e-12, atol=1e-15)
    _bf16_close(out, ref)
    assert np.abs(np.concatenate(list(ys.values()))).max() > 0


def test_ffn_zero_gate_gives_residual():
    W = moegen.WORKLOADS["tiny"]
    L = moegen.make_layer(W)
    L.gate_q[:] = 0  # all gate weights 0 -> silu(0) = 0 -> expert output 0
    x = moegen.make_tokens(W, W.T)
    res = moegen.make_residual(W, W.T)
    _, idx, w = oracle.route(x, L)
    out = oracle.ffn_combine(L, x, idx, w, residual=res)
    assert (out == res).all()


def test_ffn_single_expert_identity():
    W = moegen.WORKLOADS["tiny"]
    L = moegen.make_layer(W)
    x = moegen.make_tokens(W, W.T)
    idx = np.array([[3], [0], [7], [3]], np.int32)
    w = np.ones((W.T, 1), np.float32)
    out, y = oracle.ffn_combine(L, x, idx, w, want_y=True)
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    # y is double; rounding it through fp32 first may differ by one bf16 ulp at ties only
    _bf16_close(out, y, ulps=1)
    assert np.mean(out.view(np.int16) == ref) > 0.99


def test_expert_rows_equals_expert():
    """The batched evaluation runs the same sums in the same order as the
    per-row oracle: equal bit for bit, for every down format."""
    for fmt in (moegen.FMT_NVFP4, moegen.FMT_Q6K, moegen.FMT_Q8_0):
        w = moegen.Workload(name="rows", E=3, k=2, H=256, I=256, T=5, fmt_down=fmt)
        L = moegen.make_layer(w)
        x = moegen.make_tokens(w, 5)
        a = oracle.expert_rows(L, 2, x)
        b = np.stack([oracle.expert(L, 2, x[i]) for i in range(5)])
        assert np.array_equal(a, b)


def test_openmp_timing_build_gives_the_same_results():
    """The all-cores build of the oracle (CPU baseline timing only) computes
    the same expert outputs and layer output bit for bit."""
    w = moegen.Workload(name="omp", E=16, k=4, H=256, I=256, T=9)
    L = moegen.make_layer(w)
    x = moegen.make_tokens(w, 9)
    res = moegen.make_residual(w, 9)
    logits, idx, wt = oracle.route(x, L)
    a, ya = oracle.ffn_combine(L, x, idx, wt, res, want_y=True)
    b, yb = oracle.ffn_combine(L, x, idx, wt, res, want_y=True, parallel=True)
    assert np.array_equal(a, b) and np.array_equal(ya, yb)
    toks = [1, 4, 8]
    c = oracle.ffn_combine(L, x, idx, wt, None, toks, parallel=True)
    assert np.array_equal(c[toks], oracle.ffn_combine(L, x, idx, wt, None, toks)[toks])


# ---------------------------------------------------------------- IQ3-style grid

def _grid_by_sorting():
    """The grid's definition by brute force: all 8^4 vectors of odd integers
    1..15, sorted by (squared norm, lexicographic), the first 256."""
    odd = range(1, 16, 2)
    allv = sorted(itertools.product(odd, repeat=4), key=lambda v: (sum(c * c for c in v), v))
    return np.array(allv[:256], np.uint8)


def test_iq3g_grid_is_the_256_smallest_odd_vectors():
    """The oracle's grid (built by walking norms upward) equals the sorted
    brute-force enumeration; its shells are whole up to norm 108 (247
    vectors), and the last 9 entries are the lexicographically first of norm
    116, so the largest magnitude is 9."""
    g = oracle.iq3g_grid()
    np.testing.assert_array_equal(g, _grid_by_sorting())
    norms = (g.astype(np.int64) ** 2).sum(1)
    assert len({tuple(v) for v in g}) == 256
    assert (np.diff(norms) >= 0).all() and (g % 2 == 1).all()
    assert (norms <= 108).sum() == 247 and (norms == 116).sum() == 9
    n108 = sum(1 for v in itertools.product(range(1, 16, 2), repeat=4)
               if sum(c * c for c in v) <= 108)
    assert n108 == 247
    assert g.max() == 9 and tuple(g[0]) == (1, 1, 1, 1)


def test_iq3g_decode_closed_form():
    """Blocks packed by the documented byte layout from random integers:
    decode equals d * (2 s + 1) * grid[idx][k % 4] * sign, with the grid from
    the brute-force enumeration and d from numpy's float16."""
    rng = np.random.default_rng(11)
    G = _grid_by_sorting().astype(np.float64)
    N, K = 3, 512
    nb = K // 256
    d = (rng.standard_normal((N, nb)) * 1e-3).astype(np.float16)
    s = rng.integers(0, 16, size=(N, K // 32))
    idx = rng.integers(0, 256, size=(N, K // 4))
    neg = rng.integers(0, 2, size=(N, K))
    blocks = np.zeros((N, nb, 102), np.uint8)
    for n in range(N):
        for b in range(nb):
            blocks[n, b, 0:2] = np.frombuffer(d[n, b].tobytes(), np.uint8)
            for j in range(8):
                blocks[n, b, 2 + j // 2] |= s[n, 8 * b + j] << (4 * (j % 2))
            blocks[n, b, 6:70] = idx[n, 64 * b:64 * b + 64]
            for r in range(256):
                blocks[n, b, 70 + r // 8] |= neg[n, 256 * b + r] << (r % 8)
    got = oracle.decode_iq3g(blocks.reshape(N, -1), K)
    for n in range(N):
        for k in range(K):
            exp = float(d[n, k // 256]) * (2 * s[n, k // 32] + 1) * G[idx[n, k // 4], k % 4]
            assert got[n, k] == (-exp if neg[n, k] else exp)


def test_iq3g_generator_roundtrip_on_grid():
    """Weights that are exactly d * (2 s_j + 1) * (grid vector) * sign, with
    d = 2^-10, one sub-block at s = 15 and a magnitude 9 in every sub-block
    (so the quantizer's unit amax / 9 and scale max / 31 are exact), survive
    quantize -> decode exactly; an all-zero superblock decodes to zeros."""
    rng = np.random.default_rng(12)
    G = _grid_by_sorting().astype(np.float64)
    nine = np.flatnonzero((G == 9).any(1))
    N, K = 2, 512
    W = np.zeros((N, K))
    for n in range(N):
        for j in range(K // 32):
            sj = 15 if j % 8 == 0 else int(rng.integers(0, 16))
            unit = 2.0 ** -10 * (2 * sj + 1)
            for g in range(8):
                e = int(nine[rng.integers(len(nine))]) if g == 0 else int(rng.integers(256))
                sign = np.where(rng.integers(0, 2, 4) > 0, -1.0, 1.0)
                W[n, 32 * j + 4 * g:32 * j + 4 * g + 4] = unit * G[e] * sign
    W[1, 256:] = 0.0
    W = W.astype(np.float32)
    assert (W.astype(np.float64) == W).all()
    dec = oracle.decode_iq3g(moegen.quant_iq3g(W), K)
    np.testing.assert_array_equal(dec, W.astype(np.float64))


def test_iq3g_generator_signs_and_error_bound():
    """On Gaussian weights every nonzero decoded weight keeps the input's
    sign, and each group's decoded vector is the grid entry (times its unit)
    nearest to the input whenever the input's nearest odd magnitudes form a
    grid vector."""
    rng = np.random.default_rng(13)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    q = moegen.quant_iq3g(W)
    dec = oracle.decode_iq3g(q, 256)
    nz = dec != 0
    assert (np.sign(dec[nz]) == np.sign(W[nz])).all()
    G = _grid_by_sorting()
    gset = {tuple(v) for v in G}
    blk = q.reshape(4, 102)
    d = blk[:, :2].copy().view(np.float16).astype(np.float64)[:, 0]
    checked = 0
    for n in range(4):
        for g in range(64):
            j = g // 8
            s = (blk[n, 2 + j // 2] >> (4 * (j % 2))) & 15
            unit = d[n] * (2 * int(s) + 1)
            t = np.abs(W[n, 4 * g:4 * g + 4].astype(np.float64)) / unit
            m = np.clip(2 * np.rint((t - 1) / 2) + 1, 1, 15).astype(int)
            if tuple(m) in gset:
                np.testing.assert_array_equal(np.abs(dec[n, 4 * g:4 * g + 4]), unit * m)
                checked += 1
    assert checked > 200


def _ternary_grid_by_sorting():
    allv = sorted(itertools.product((-1, 0, 1), repeat=8),
                  key=lambda v: (sum(c != 0 for c in v), v))
    return np.array(allv[:1024], np.int8)


def test_iq1g_grid_is_the_1024_sparsest_ternary_vectors():
    """The oracle's grid (built by walking nonzero counts upward) equals the
    sorted brute-force enumeration of {-1, 0, +1}^8: every vector with at
    most 3 nonzero values (1 + 16 + 112 + 448 = 577), then the first 447 with
    4 in lexicographic order."""
    g = oracle.iq1g_grid()
    np.testing.assert_array_equal(g, _ternary_grid_by_sorting())
    nz = (g != 0).sum(1)
    assert [int((nz == c).sum()) for c in range(5)] == [1, 16, 112, 448, 447]
    assert (np.diff(nz) >= 0).all() and len({tuple(v) for v in g}) == 1024
    assert tuple(g[0]) == (0,) * 8 and tuple(g[1]) == (-1,) + (0,) * 7
    assert tuple(g[9]) == (0,) * 7 + (1,) and tuple(g[16]) == (1,) + (0,) * 7
    assert tuple(g[577]) == (-1, -1, -1, -1, 0, 0, 0, 0)
    assert int(np.abs(g).max()) == 1


def test_iq1g_decode_closed_form():
    """Blocks packed by the documented byte layout from random integers:
    decode equals d * (2 s + 1) * grid[idx][k % 8], with the grid from the
    brute-force enumeration, the 10-bit index split into its low byte and
    2-bit high part, and d from numpy's float16."""
    rng = np.random.default_rng(21)
    G = _ternary_grid_by_sorting().astype(np.float64)
    N, K = 3, 512
    nb = K // 256
    d = (rng.standard_normal((N, nb)) * 1e-3).astype(np.float16)
    s = rng.integers(0, 16, size=(N, K // 32))
    idx = rng.integers(0, 1024, size=(N, K // 8))
    blocks = np.zeros((N, nb, 46), np.uint8)
    for n in range(N):
        for b in range(nb):
            blocks[n, b, 0:2] = np.frombuffer(d[n, b].tobytes(), np.uint8)
            for j in range(8):
                blocks[n, b, 2 + j // 2] |= s[n, 8 * b + j] << (4 * (j % 2))
            for g in range(32):
                i = idx[n, 32 * b + g]
                blocks[n, b, 6 + g] = i & 255
                blocks[n, b, 38 + g // 4] |= (i >> 8) << (2 * (g % 4))
    got = oracle.decode_iq1g(blocks.reshape(N, -1), K)
    for n in range(N):
        for k in range(K):
            exp = float(d[n, k // 256]) * (2 * s[n, k // 32] + 1) * G[idx[n, k // 8], k % 8]
            assert got[n, k] == exp


def test_iq1g_generator_roundtrip_on_grid():
    """Weights that are exactly d * (2 s_j + 1) * (grid vector), d = 2^-10,
    one sub-block at s = 15 and a nonzero value in every sub-block (so the
    quantizer's unit amax and scale max / 31 are exact), survive quantize ->
    decode exactly; an all-zero superblock decodes to zeros."""
    rng = np.random.default_rng(22)
    G = _ternary_grid_by_sorting().astype(np.float64)
    N, K = 2, 512
    W = np.zeros((N, K))
    for n in range(N):
        for j in range(K // 32):
            sj = 15 if j % 8 == 0 else int(rng.integers(0, 16))
            unit = 2.0 ** -10 * (2 * sj + 1)
            for g in range(4):
                e = int(rng.integers(1, 1024)) if g == 0 else int(rng.integers(1024))
                W[n, 32 * j + 8 * g:32 * j + 8 * g + 8] = unit * G[e]
    W[1, 256:] = 0.0
    W = W.astype(np.float32)
    assert (W.astype(np.float64) == W).all()
    q = moegen.quant_iq1g(W)
    np.testing.assert_array_equal(oracle.decode_iq1g(q, K), W.astype(np.float64))


def test_iq1g_generator_keeps_signs_and_rounds_in_grid():
    """On Gaussian weights every nonzero decoded weight keeps the input's
    sign and is one unit in magnitude, and a group whose rounded vector has at
    most 3 nonzero values (always in the grid) decodes to exactly that
    rounding."""
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((4, 256)) * 0.02).astype(np.float32)
    q = moegen.quant_iq1g(W)
    dec = oracle.decode_iq1g(q, 256)
    nz = dec != 0
    assert nz.any() and (np.sign(dec[nz]) == np.sign(W[nz])).all()
    blk = q.reshape(4, 46)
    d = blk[:, :2].copy().view(np.float16).astype(np.float64)[:, 0]
    checked = 0
    for n in range(4):
        for g in range(32):
            j = g // 4
            sj = (int(blk[n, 2 + j // 2]) >> (4 * (j % 2))) & 15
            unit = d[n] * (2 * sj + 1)
            t = W[n, 8 * g:8 * g + 8].astype(np.float64) / unit
            r = np.where(np.abs(t) >= 0.5, np.sign(t), 0.0)
            np.testing.assert_array_equal(np.abs(dec[n, 8 * g:8 * g + 8]) <= unit, True)
            if (r != 0).sum() <= 3:
                np.testing.assert_array_equal(dec[n, 8 * g:8 * g + 8], r * unit)
                checked += 1
    assert checked > 64
