"""Router logits and top-k (moe_route) against the oracle, bit for bit, on
shapes that reach every edge of the multi-token router kernel: H in one or
several 2048-wide chunks, expert counts that leave whole waves without
experts, token counts that end inside an 8-token block, a router bias, and the
boundary with the one-pair-per-wave kernel used at decode sizes."""
import numpy as np
import pytest
import torch

import moegen
import quantized_expert_ffn_router_amd as q
from parity_util import check_route

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,E,k,H,zipf", [
    (64, 128, 8, 2048, 0.0),    # largest decode-size batch
    (65, 40, 4, 4096, 0.0),     # two H chunks; waves past E = 40; 1 token in the last block
    (130, 128, 8, 2048, 1.1),   # router bias; 2 tokens in the last block
    (77, 1024, 8, 128, 0.0),    # one 128-wide chunk; 32 expert groups
    (200, 8, 2, 8192, 0.0),     # four chunks; three of four waves without experts
    (1029, 256, 8, 2048, 1.1),  # 129 token blocks: a partial group of eight blocks
])
def test_router_logits_bit_exact(T, E, k, H, zipf):
    w = moegen.Workload(name="router", E=E, k=k, H=H, I=128, T=T, zipf_s=zipf,
                        zipf_alpha=1.0 if zipf else 0.0)
    L = moegen.make_layer(w)
    assert (L.bias is not None) == (zipf > 0)
    x = moegen.make_tokens(w, T, step=3)
    print("router", T, E, k, H, zipf, flush=True)
    dl = q.DeviceLayer(L)
    buf = q.StepBuffers(dl, T)
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    buf.logits.fill_(float("nan"))
    q.moe_route(dl.desc, xd, T, buf.logits, buf.idx, buf.w)
    torch.cuda.synchronize()
    g = dict(logits=buf.logits[:T].cpu().numpy(), idx=buf.idx[:T].cpu().numpy(),
             w=buf.w[:T].cpu().numpy())
    check_route(g, L, x)


@pytest.mark.parametrize("T", [4, 70])
def test_topk_ties_across_lanes_and_slots(T):
    """Zero router weights and a crafted bias: every token's logits equal the
    bias, with equal values at experts in different 64-expert slots and
    lanes (ties go to the lower index), negative values and values that
    differ in the last bit.  T = 4 takes the fused gating kernel, T = 70 the
    separate top-k."""
    E, k = 200, 8
    w = moegen.Workload(name="ties", E=E, k=k, H=256, I=128, T=T)
    L = moegen.make_layer(w)
    bias = np.full(E, -5.0, np.float32)
    for e in (150, 70, 5, 199):
        bias[e] = 3.0
    for e in (128, 64, 63):
        bias[e] = 2.5
    bias[100] = np.nextafter(np.float32(2.5), np.float32(0))
    bias[1] = -1.0
    bias[130] = -1.0
    L0 = moegen.LayerWeights(**{**L.__dict__, "w_router": np.zeros_like(L.w_router), "bias": bias})
    x = moegen.make_tokens(w, T)
    dl = q.DeviceLayer(L0)
    buf = q.StepBuffers(dl, T)
    xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
    if T <= 64:
        q.moe_route_bucket(dl.desc, xd, T, buf.logits, buf.idx, buf.w, buf.buckets, buf.ws,
                           buf.ws_bytes, buf.hist, 5, 10)
    else:
        q.moe_route(dl.desc, xd, T, buf.logits, buf.idx, buf.w)
    torch.cuda.synchronize()
    g = dict(logits=buf.logits[:T].cpu().numpy(), idx=buf.idx[:T].cpu().numpy(),
             w=buf.w[:T].cpu().numpy())
    check_route(g, L0, x)
    assert (g["idx"] == np.array([5, 70, 150, 199, 63, 64, 128, 100])).all()
