"""moe_route_bucket (router logits, then top-k + bucketing + histogram in one
launch for decode sizes) against moe_route + moe_bucket + moe_expert_hist on
the same inputs: every output bit-identical, on both sides of the fused
kernel's limits (E <= 256, T*k <= 256) and against the oracle."""
import numpy as np
import pytest
import torch

import moegen
import oracle
import quantized_expert_ffn_router_amd as q
from parity_util import check_buckets, check_route

pytestmark = pytest.mark.gpu


def _run(L, x, fused, hist0, with_hist=True):
    T = x.shape[0]
    dl = q.DeviceLayer(L)
    buf = q.StepBuffers(dl, max(T, 1))
    buf.hist.copy_(torch.from_numpy(hist0.view(np.int32)).cuda())
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    d = dl.desc
    if fused:
        q.moe_route_bucket(d, xd, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws, buf.ws_bytes,
                           buf.hist if with_hist else None, 5, 10)
    else:
        q.moe_route(d, xd, T, buf.logits, buf.idx, buf.w)
        q.moe_bucket(d, buf.idx, T, buf.buckets, buf.ws, buf.ws_bytes)
        if with_hist:
            q.moe_expert_hist(d, buf.buckets, buf.hist, 5, 10)
    torch.cuda.synchronize()
    return dict(logits=buf.logits[:T].cpu().numpy(), idx=buf.idx[:T].cpu().numpy(),
                w=buf.w[:T].cpu().numpy(), buckets=buf.bucket_view(L.E, T, L.k),
                hist=buf.hist.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("E,k,H,T,renorm", [
    (8, 2, 256, 4, 1),
    (128, 8, 2048, 1, 1),
    (128, 8, 2048, 8, 1),
    (128, 8, 512, 32, 1),    # T*k = 256: the largest fused case
    (256, 1, 256, 64, 1),    # T = 64: the widest token mask
    (256, 1, 256, 65, 1),    # T = 65: separate kernels
    (128, 8, 512, 33, 1),    # T*k = 264: separate kernels
    (256, 8, 512, 8, 1),
    (512, 4, 256, 8, 1),     # E > 256: separate kernels
    (64, 64, 256, 3, 0),     # k = E, full softmax
])
def test_fused_gating_equals_separate_calls(E, k, H, T, renorm):
    w = moegen.Workload(name="gate", E=E, k=k, H=H, I=128, T=T, renormalize=renorm)
    L = moegen.make_layer(w)
    L.renormalize = renorm
    x = moegen.make_tokens(w, T, step=7)
    hist0 = (np.arange(E, dtype=np.uint32) * 977 + 12345).astype(np.uint32)
    a = _run(L, x, True, hist0)
    b = _run(L, x, False, hist0)
    for key in ("logits", "idx", "w", "hist"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    for key in ("counts", "offsets", "sorted_asg", "asg_pos", "active"):
        assert np.array_equal(a["buckets"][key], b["buckets"][key]), key
    assert a["buckets"]["n_active"] == b["buckets"]["n_active"]
    # and both against the oracle
    logits, idx, wt = check_route(a, L, x)
    ob = check_buckets(a["buckets"], idx, E)
    assert np.array_equal(a["hist"], oracle.hist(ob["counts"], hist0, 5, 10))


def test_fused_gating_without_histogram_leaves_it():
    w = moegen.Workload(name="gate", E=128, k=8, H=512, I=128, T=8)
    L = moegen.make_layer(w)
    x = moegen.make_tokens(w, 8, step=2)
    hist0 = np.full(128, 7, np.uint32)
    a = _run(L, x, True, hist0, with_hist=False)
    assert np.array_equal(a["hist"], hist0)
