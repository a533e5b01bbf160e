"""moe_expert_ffn_noalloc: the expert FFN with the library's static per-GPU
workspace instead of a caller workspace.  Called through the C ABI and
compared bit for bit with moe_expert_ffn on a caller workspace, three calls in
a row on one GPU, each smaller than the one before (grouped GEMM at 600 and
300 tokens, then the decode GEMV at 5), so each call runs on what the
previous one left in the shared buffer; a call beyond the buffer is refused
before any launch."""
import numpy as np
import pytest

import moegen
from parity_util import check_y_rows, oracle_y

pytestmark = pytest.mark.gpu


def _ffn_both_ways(q, torch, dl, w, T, step, y_dtype):
    buf = q.StepBuffers(dl, T, y_dtype)
    x = moegen.make_tokens(w, T, step=step)
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    q.moe_route_bucket(dl.desc, xd, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                       buf.ws_bytes)
    q.moe_expert_ffn(dl.desc, xd, T, buf.buckets, buf.y, y_dtype, buf.ws, buf.ws_bytes)
    torch.cuda.synchronize()
    ref = buf.y[:T * w.k].clone()
    buf.y.fill_(float("nan"))
    q.moe_expert_ffn_noalloc(dl.desc, xd, T, buf.buckets, buf.y, y_dtype)
    torch.cuda.synchronize()
    got = buf.y[:T * w.k].clone()
    return x, buf, ref, got


def test_noalloc_ffn_equals_workspace_ffn_on_successive_smaller_calls():
    import torch
    import quantized_expert_ffn_router_amd as q
    w = moegen.Workload(name="noalloc", E=64, k=8, H=256, I=128, T=600)
    L = moegen.make_layer(w)
    dl = q.DeviceLayer(L)
    for T, step, y_dtype in [(600, 1, 0), (300, 2, 1), (5, 3, 0)]:
        print("noalloc T", T, "y_dtype", y_dtype, flush=True)
        x, buf, ref, got = _ffn_both_ways(q, torch, dl, w, T, step, y_dtype)
        assert torch.equal(got.view(torch.int16) if y_dtype else got.view(torch.int32),
                           ref.view(torch.int16) if y_dtype else ref.view(torch.int32)), T
        # and against the oracle, on the first and last assignment of each token block
        bk = buf.bucket_view(w.E, T, w.k)
        rows = np.unique(np.r_[0:T * w.k:7, T * w.k - 1])
        idx = buf.idx[:T].cpu().numpy()
        oy = oracle_y(L, x, idx, bk["sorted_asg"][rows])
        check_y_rows(got.float().cpu().numpy()[rows], oy)


def test_noalloc_ffn_refuses_calls_beyond_its_buffer():
    import torch
    import quantized_expert_ffn_router_amd as q
    w = moegen.Workload(name="noalloc", E=64, k=8, H=256, I=128, T=16384)
    dl = q.DeviceLayer(moegen.make_layer(w))
    T = 16384
    buf = q.StepBuffers(dl, T, 1)
    assert q.moe_workspace_bytes(dl.desc, T) > q.MOE_NOALLOC_WORKSPACE_BYTES
    xd = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
    with pytest.raises(q.MoeError) as ei:
        q.moe_expert_ffn_noalloc(dl.desc, xd, T, buf.buckets, buf.y, 1)
    assert ei.value.status == q.MOE_ERR_WORKSPACE
    assert "static" in q.last_error()
