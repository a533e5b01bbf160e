"""moe_route_ffn: routing, gating, bucketing, histogram and the expert FFN
in one call, which for batches of up to 4 tokens runs the gating inside the gate/up
kernel (every workgroup repeats it in LDS; one writes the outputs).  Called
through the C ABI and compared bit for bit with moe_route_bucket followed by
moe_expert_ffn on the same inputs: logits, top-k indices and weights, every
bucket array, the histogram and the expert outputs y; larger batches (the
two calls inside) are compared too."""
import numpy as np
import pytest

import moegen

pytestmark = pytest.mark.gpu

CASES = [  # (workload or shape, T values: up to 4 one launch fewer, then the two calls)
    ("decode", None, (1, 2, 4, 5, 8)),
    ("wide", dict(E=256, k=8, H=1024, I=512, T=16), (3, 16)),       # 4 logits per lane
    ("narrow", dict(E=64, k=4, H=512, I=256, T=16), (1, 7)),        # 1 logit per lane
    ("mixed", None, (4, 8)),                                       # Q6_K down
    ("iq1", None, (3,)),                                           # IQ1G down
    ("biased", dict(E=128, k=8, H=512, I=256, T=16, zipf_s=1.1, zipf_alpha=0.44), (4, 6)),
    ("full_softmax", dict(E=32, k=2, H=256, I=128, T=16, renormalize=0), (2, 9)),
]


def _workload(name, over):
    if over is None:
        return moegen.WORKLOADS[name]
    return moegen.Workload(name=name, **over)


def _run(q, torch, dl, xd, T, fused, y_dtype):
    buf = q.StepBuffers(dl, T, y_dtype)
    buf.hist.copy_(torch.arange(dl.E, dtype=torch.int32, device="cuda") * 1000)
    if fused:
        q.moe_route_ffn(dl.desc, xd, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.hist, 5, 10,
                        buf.y, y_dtype, buf.ws, buf.ws_bytes)
    else:
        q.moe_route_bucket(dl.desc, xd, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                           buf.ws_bytes, buf.hist, 5, 10)
        q.moe_expert_ffn(dl.desc, xd, T, buf.buckets, buf.y, y_dtype, buf.ws, buf.ws_bytes)
    torch.cuda.synchronize()
    A = T * dl.k
    bk = buf.bucket_view(dl.E, T, dl.k)
    return dict(logits=buf.logits[:T].cpu().numpy().view(np.uint32),
                idx=buf.idx[:T].cpu().numpy(), w=buf.w[:T].cpu().numpy().view(np.uint32),
                hist=buf.hist.cpu().numpy(),
                y=buf.y[:A].view(torch.int16 if y_dtype else torch.int32).cpu().numpy(), **bk)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_route_ffn_equals_route_bucket_then_ffn(case):
    import torch
    import quantized_expert_ffn_router_amd as q
    name, over, Ts = case
    w = _workload(name, over)
    dl = q.DeviceLayer(moegen.make_layer(w))
    for T in Ts:
        for y_dtype in (0, 1):
            print("route_ffn", name, "T", T, "y_dtype", y_dtype, flush=True)
            x = moegen.make_tokens(w, T, step=T + 40)
            xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
            ref = _run(q, torch, dl, xd, T, False, y_dtype)
            got = _run(q, torch, dl, xd, T, True, y_dtype)
            for key in ref:
                a, b = np.asarray(got[key]), np.asarray(ref[key])
                assert a.shape == b.shape and np.array_equal(a, b), (name, T, y_dtype, key)
