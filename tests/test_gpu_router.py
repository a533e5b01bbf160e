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
