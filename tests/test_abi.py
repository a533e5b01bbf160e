"""C-ABI contract checks that need no GPU: the library loads, exports every
entry point declared in include/moe.h, and rejects bad arguments on the host
before any launch (these paths never touch the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_expert_ffn_router_amd as q
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (moe_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = q.lib()
    for n in names:
        assert hasattr(lib, n)
    assert set(q.SIGNATURES) == set(names)


def test_abi_version_and_struct_sizes():
    assert q.moe_abi_version() == 2
    src = open(HEADER).read()
    assert "#define MOE_ABI_VERSION 2" in src
    assert ctypes.sizeof(q.ExpertRef) == 24


def test_blob_sizes():
    # codes + scales of gate, up, down: 3 * I*H*(1/2 + 1/16)
    assert q.moe_expert_blob_bytes(2048, 768, 1, 1) == 3 * (768 * 2048 // 2 + 768 * 2048 // 16)
    # Q6_K down: 210 bytes per 256 weights, plus the 256-byte exponent section
    assert q.moe_expert_blob_bytes(2048, 512, 1, 2) == 2 * (512 * 2048 * 9 // 16) + 2048 * 2 * 210 + 256
    assert q.moe_expert_blob_bytes(100, 768, 1, 1) == 0
    assert "multiple of 128" in q.last_error()
    assert q.moe_expert_blob_bytes(2048, 384, 1, 2) == 0  # Q6_K needs I % 256


def _desc(E=8, k=2, H=256, I=128, fmt_down=1, renorm=1, ffn_mode=0):
    return q.LayerDesc(E, k, H, I, 1, fmt_down, renorm, ffn_mode, 0x1000, 0x2000, None)


def test_buckets_carve_layout_on_host_buffer():
    E, T, k = 128, 8, 8
    n = q.moe_buckets_bytes(E, T, k)
    buf = np.zeros(n + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    b = q.moe_buckets_carve(base, n, E, T, k)
    assert b.counts == base and b.T_max == T and b.E == E and b.k == k
    ptrs = [b.counts, b.offsets, b.sorted_asg, b.asg_pos, b.active, b.n_active]
    assert ptrs == sorted(ptrs) and all(p % 256 == 0 for p in ptrs)
    assert b.n_active + 4 <= base + n
    with pytest.raises(q.MoeError) as ei:
        q.moe_buckets_carve(base, n - 1, E, T, k)
    assert ei.value.status == q.MOE_ERR_WORKSPACE
    with pytest.raises(q.MoeError) as ei:
        q.moe_buckets_carve(base + 4, n, E, T, k)
    assert ei.value.status == q.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status,msg", [
    (dict(k=9), q.MOE_ERR_INVALID_ARG, "k=9 > E=8"),
    (dict(E=2000, k=2), q.MOE_ERR_UNSUPPORTED, "E=2000"),
    (dict(E=128, k=65), q.MOE_ERR_UNSUPPORTED, "k=65"),
    (dict(H=200), q.MOE_ERR_UNSUPPORTED, "H=200"),
    (dict(I=100), q.MOE_ERR_UNSUPPORTED, "I=100"),
    (dict(I=384, fmt_down=2), q.MOE_ERR_UNSUPPORTED, "Q6_K"),
    (dict(I=96, fmt_down=3), q.MOE_ERR_UNSUPPORTED, "I=96"),
    (dict(I=384, fmt_down=4), q.MOE_ERR_UNSUPPORTED, "I=384"),
    (dict(fmt_down=7), q.MOE_ERR_UNSUPPORTED, "down format"),
    (dict(renorm=2), q.MOE_ERR_INVALID_ARG, "renormalize"),
    (dict(ffn_mode=3), q.MOE_ERR_INVALID_ARG, "ffn_mode=3"),
    (dict(ffn_mode=-1), q.MOE_ERR_INVALID_ARG, "ffn_mode=-1"),
])
def test_route_rejects_bad_layers_before_launch(kw, status, msg):
    d = _desc(**kw)
    st = q.lib().moe_route(ctypes.byref(d), 0x10, 4, 0x20, 0x30, 0x40, None)
    assert st == status
    assert msg in q.last_error()


def test_zero_tokens_is_a_noop_and_null_checks():
    d = _desc()
    lib = q.lib()
    assert lib.moe_route(ctypes.byref(d), None, 0, None, None, None, None) == q.MOE_OK
    assert lib.moe_route(ctypes.byref(d), 0x10, -1, 0x20, 0x30, 0x40, None) == q.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(d), None, 4, 0x20, 0x30, 0x40, None) == q.MOE_ERR_INVALID_ARG
    assert "x is NULL" in q.last_error()
    n = q.moe_buckets_bytes(8, 4, 2)
    buf = np.zeros(n + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    b = q.moe_buckets_carve(base, n, 8, 4, 2)
    assert lib.moe_bucket(ctypes.byref(d), None, 0, ctypes.byref(b), None, 0, None) == q.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(d), None, 0, ctypes.byref(b), None, 0, None, 0, None) == q.MOE_OK
    assert lib.moe_combine(ctypes.byref(d), None, 0, ctypes.byref(b), None, 0, None, None, None) == q.MOE_OK
    # capacity and carve mismatch
    assert lib.moe_bucket(ctypes.byref(d), 0x10, 5, ctypes.byref(b), None, 0, None) == q.MOE_ERR_WORKSPACE
    d2 = _desc(E=16)
    assert lib.moe_bucket(ctypes.byref(d2), 0x10, 4, ctypes.byref(b), None, 0, None) == q.MOE_ERR_INVALID_ARG
    # ffn workspace too small, bad y dtype
    assert lib.moe_expert_ffn(ctypes.byref(d), 0x10, 4, ctypes.byref(b), 0x20, 0, 0x30, 16, None) == q.MOE_ERR_WORKSPACE
    assert lib.moe_expert_ffn(ctypes.byref(d), 0x10, 4, ctypes.byref(b), 0x20, 5, 0x30, 1 << 20, None) == q.MOE_ERR_INVALID_ARG
    # histogram shift range
    assert lib.moe_expert_hist(ctypes.byref(d), ctypes.byref(b), 0x10, 40, 10, None) == q.MOE_ERR_INVALID_ARG


def test_blob_bytes_per_down_format():
    """Sections start on 256-byte boundaries: gate and up (NVFP4 codes and
    scales), then the down projection's planes; Q6_K, Q8_0, IQ3G and IQ1G blobs end
    with a 256-byte section for the grouped GEMM's per-expert weight
    exponent."""
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    H, I = 2048, 768
    gu = 2 * (al(I * H // 2) + al(I * H // 16))
    assert q.moe_expert_blob_bytes(H, I, 1, 1) == gu + al(H * I // 2) + al(H * I // 16)
    assert q.moe_expert_blob_bytes(H, I, 1, 3) == gu + al(H * I) + al(H * I // 16) + 256
    I = 512
    gu = 2 * (al(I * H // 2) + al(I * H // 16))
    assert q.moe_expert_blob_bytes(H, I, 1, 2) == gu + al(H * I // 2) + al(H * I // 4) + \
        al(H * I // 16) + al(H * I // 128) + 256
    assert q.moe_expert_blob_bytes(H, 96, 1, 3) == 0
    # IQ3G: grid indices (I/4 per row), sign bits (I/8), d and multipliers
    # (8 bytes per 256), exponent section
    assert q.moe_expert_blob_bytes(H, I, 1, 4) == gu + al(H * I // 4) + al(H * I // 8) + \
        al(H * I // 32) + 256
    assert q.moe_expert_blob_bytes(H, 384, 1, 4) == 0
    # IQ1G: index low bytes (I/8 per row), 2-bit high parts (I/32), d and
    # multipliers (8 bytes per 256), exponent section
    assert q.moe_expert_blob_bytes(H, I, 1, 5) == gu + al(H * I // 8) + al(H * I // 32) + \
        al(H * I // 32) + 256
    assert q.moe_expert_blob_bytes(H, 384, 1, 5) == 0
    assert "IQ1G" in q.last_error()


def test_workspace_bytes_cover_hidden_buffers():
    d = _desc(E=128, k=8, H=2048, I=768)
    # h (bf16 [T*k][I]) + fp16 copy of x ([T][H]) + its row scales + the
    # grouped GEMM's row-block tables (>= one 128-entry table per block)
    T = 16384
    ws = q.moe_workspace_bytes(d, T)
    blocks = T * 8 // 128
    assert ws >= T * 8 * 768 * 2 + T * 2048 * 2 + T * 4 + blocks * 128 * 8
    assert q.moe_workspace_bytes(d, 1) >= 8 * 768 * 2 + 2048 * 2 + 4


def test_tier_create_rejects_small_budget_before_any_hip_call():
    E, L, R, S, eb = 8, 2, 4, 2, 1024
    ptrs = (ctypes.c_void_p * (L * E))(*([0x1000] * (L * E)))
    scales = (q.ExpertRef * (L * E))()
    desc = q.TierDesc(L, E, R, S, eb, ctypes.addressof(ptrs), ctypes.addressof(scales), 0x100000,
                      (L * R + S) * eb - 1, None)
    with pytest.raises(q.MoeError) as ei:
        q.moe_tier_create(desc)
    assert ei.value.status == q.MOE_ERR_BUDGET
    assert "HBM pool" in q.last_error()
    desc.resident_per_layer = E + 1
    with pytest.raises(q.MoeError) as ei:
        q.moe_tier_create(desc)
    assert ei.value.status == q.MOE_ERR_INVALID_ARG


def test_route_bucket_checks_before_launch():
    d = _desc()
    lib = q.lib()
    n = q.moe_buckets_bytes(8, 4, 2)
    buf = np.zeros(n + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    b = q.moe_buckets_carve(base, n, 8, 4, 2)
    f = lib.moe_route_bucket
    assert f(ctypes.byref(d), None, 0, None, None, None, ctypes.byref(b), None, 0, None, 0, 0,
             None) == q.MOE_OK
    assert f(ctypes.byref(d), None, 4, 0x20, 0x30, 0x40, ctypes.byref(b), None, 0, None, 0, 0,
             None) == q.MOE_ERR_INVALID_ARG
    assert "x is NULL" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, 0x20, 0x30, 0x40, ctypes.byref(b), None, 0, 0x50, 40, 10,
             None) == q.MOE_ERR_INVALID_ARG
    assert "shifts" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 5, 0x20, 0x30, 0x40, ctypes.byref(b), None, 0, None, 0, 0,
             None) == q.MOE_ERR_WORKSPACE


def test_route_ffn_checks_before_launch():
    """moe_route_ffn validates everything on the host first: zero tokens is a
    no-op; null pointers, histogram shifts, the y type, capacity and the
    workspace size are refused before any launch."""
    d = _desc()
    lib = q.lib()
    n = q.moe_buckets_bytes(8, 4, 2)
    buf = np.zeros(n + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    b = q.moe_buckets_carve(base, n, 8, 4, 2)
    f = lib.moe_route_ffn
    B = ctypes.byref(b)
    big = 1 << 20
    assert f(ctypes.byref(d), None, 0, None, None, None, B, None, 0, 0, None, 0, None, 0,
             None) == q.MOE_OK
    assert f(ctypes.byref(d), None, 4, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0, 0x70, big,
             None) == q.MOE_ERR_INVALID_ARG
    assert "x is NULL" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, None, 0x30, 0x40, B, None, 0, 0, 0x60, 0, 0x70, big,
             None) == q.MOE_ERR_INVALID_ARG
    assert "logits is NULL" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, 0x20, 0x30, 0x40, B, 0x50, 40, 10, 0x60, 0, 0x70, big,
             None) == q.MOE_ERR_INVALID_ARG
    assert "shifts" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 7, 0x70, big,
             None) == q.MOE_ERR_INVALID_ARG
    assert "y_dtype" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 5, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0, 0x70, big,
             None) == q.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(d), 0x10, 4, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0, 0x70, 16,
             None) == q.MOE_ERR_WORKSPACE


def test_layer_forward_checks_before_launch():
    """moe_layer_forward validates on the host first, like moe_route_ffn,
    and also needs the output buffer."""
    d = _desc()
    lib = q.lib()
    n = q.moe_buckets_bytes(8, 4, 2)
    buf = np.zeros(n + 256, np.uint8)
    base = (buf.ctypes.data + 255) // 256 * 256
    b = q.moe_buckets_carve(base, n, 8, 4, 2)
    f = lib.moe_layer_forward
    B = ctypes.byref(b)
    big = 1 << 20
    assert f(ctypes.byref(d), None, 0, None, None, None, None, None, B, None, 0, 0, None, 0,
             None, 0, None) == q.MOE_OK
    assert f(ctypes.byref(d), 0x10, 4, None, None, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0,
             0x70, big, None) == q.MOE_ERR_INVALID_ARG
    assert "out is NULL" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, None, 0x80, 0x20, 0x30, 0x40, B, 0x50, 32, 0, 0x60, 0,
             0x70, big, None) == q.MOE_ERR_INVALID_ARG
    assert "shifts" in q.last_error()
    assert f(ctypes.byref(d), 0x10, 4, None, 0x80, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0,
             0x70, 16, None) == q.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(d), 0x10, 5, None, 0x80, 0x20, 0x30, 0x40, B, None, 0, 0, 0x60, 0,
             0x70, big, None) == q.MOE_ERR_WORKSPACE


def test_library_grid_equals_oracle_grid():
    """The library builds the IQ3G grid at compile time (csrc/iq3g.h, a
    counting sort on the squared norm); compiled on the host here, its 256
    entries equal the oracle's (which walks the norms) and the brute-force
    definition's."""
    import os
    import subprocess
    import tempfile
    import oracle
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = os.path.join(root, "quantized_expert_ffn_router_amd", "csrc", "iq3g.h")
    src = ('#include "%s"\n#include <cstdio>\nint main() {\n'
           '  constexpr moe::Iq3gGrid g = moe::make_iq3g_grid();\n'
           '  for (int e = 0; e < 256; ++e) printf("%%u\\n", g.m[e]);\n}\n') % hdr
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "g.cpp"), "w") as f:
            f.write(src)
        subprocess.check_call(["g++", "-std=c++17", "-O1", os.path.join(d, "g.cpp"), "-o",
                               os.path.join(d, "g")])
        out = subprocess.check_output([os.path.join(d, "g")], text=True).split()
    m = np.array([int(v) for v in out], np.uint32)
    lib_grid = np.stack([(m >> (8 * c)) & 255 for c in range(4)], axis=1).astype(np.uint8)
    np.testing.assert_array_equal(lib_grid, oracle.iq3g_grid())


def test_library_iq1g_grid_equals_oracle_grid():
    """The library builds the IQ1G grid at compile time (csrc/iq1g.h, a
    counting sort on the nonzero count, 2 bits per value); compiled on the
    host here, its 1024 entries equal the oracle's (which walks the counts)."""
    import os
    import subprocess
    import tempfile
    import oracle
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    hdr = os.path.join(root, "quantized_expert_ffn_router_amd", "csrc", "iq1g.h")
    src = ('#include "%s"\n#include <cstdio>\nint main() {\n'
           '  constexpr moe::Iq1gGrid g = moe::make_iq1g_grid();\n'
           '  for (int e = 0; e < 1024; ++e) printf("%%u\\n", (unsigned)g.c[e]);\n}\n') % hdr
    with tempfile.TemporaryDirectory() as d:
        with open(os.path.join(d, "g.cpp"), "w") as f:
            f.write(src)
        subprocess.check_call(["g++", "-std=c++17", "-O1", os.path.join(d, "g.cpp"), "-o",
                               os.path.join(d, "g")])
        out = subprocess.check_output([os.path.join(d, "g")], text=True).split()
    c = np.array([int(v) for v in out], np.uint32)
    nz = np.stack([(c >> (2 * i)) & 1 for i in range(8)], axis=1)
    neg = np.stack([(c >> (2 * i + 1)) & 1 for i in range(8)], axis=1)
    assert not (neg & (1 - nz)).any()  # a negative flag only on a nonzero value
    lib_grid = (nz * np.where(neg > 0, -1, 1)).astype(np.int8)
    np.testing.assert_array_equal(lib_grid, oracle.iq1g_grid())
