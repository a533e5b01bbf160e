"""moe_layer_forward: the whole layer step in one call.  For decode batches
(2 to 8 tokens) the down projection and the gate-weighted combine run as
one kernel that writes the layer output straight from h.  Called through
the C ABI and compared with the oracle (routing bit for bit, the output at
the layer's bars) and with moe_route_ffn + moe_combine on the same inputs
(routing outputs, buckets and histogram bit for bit; the output within a
bf16 step plus the fp32 order difference: the two sum the same terms in
different orders), with and without a residual, for every down format, k
from 2 to 12, and batches of 1 and above 8 (the separate calls inside)."""
import numpy as np
import pytest

import moegen
import oracle
from parity_util import check_out, check_route

pytestmark = pytest.mark.gpu

CASES = [  # (name, workload overrides or None, batches)
    ("decode", None, (1, 2, 4, 8, 9, 16)),
    ("mixed", None, (8,)),                                               # Q6_K down
    ("q8", None, (3,)),                                                  # Q8_0 down
    ("iq3", None, (5,)),                                                 # IQ3G down
    ("iq1", None, (2,)),                                                 # IQ1G down
    ("k2", dict(E=32, k=2, H=512, I=256, T=16), (2, 9)),                 # 2 waves
    ("k12", dict(E=64, k=12, H=1024, I=512, T=16), (4,)),                # 12 slots on 8 waves
    ("wide_h", dict(E=64, k=8, H=4096, I=256, T=16), (2,)),              # 64-row gate/up
]


def _workload(name, over):
    return moegen.WORKLOADS[name] if over is None else moegen.Workload(name=name, **over)


def _run(q, torch, dl, xd, rd, T, keep_y):
    buf = q.StepBuffers(dl, T, 0)
    buf.hist.copy_(torch.arange(dl.E, dtype=torch.int32, device="cuda") * 977)
    q.layer_forward(dl, buf, xd, T, rd, keep_y=keep_y)
    torch.cuda.synchronize()
    bk = buf.bucket_view(dl.E, T, dl.k)
    return dict(logits=buf.logits[:T].cpu().numpy().view(np.uint32),
                idx=buf.idx[:T].cpu().numpy(), w=buf.w[:T].cpu().numpy().view(np.uint32),
                hist=buf.hist.cpu().numpy(), **bk), buf.out[:T].cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_layer_forward_matches_oracle_and_separate_calls(case):
    import torch
    import quantized_expert_ffn_router_amd as q
    name, over, Ts = case
    w = _workload(name, over)
    L = moegen.make_layer(w)
    dl = q.DeviceLayer(L)
    for T in Ts:
        for with_res in (False, True):
            print("layer_forward", name, "T", T, "residual", with_res, flush=True)
            x = moegen.make_tokens(w, T, step=T + 60)
            res = moegen.make_residual(w, T, step=T) if with_res else None
            xd = torch.from_numpy(x.view(np.int16).copy()).cuda()
            rd = None if res is None else torch.from_numpy(res.view(np.int16).copy()).cuda()
            ref, out_ref = _run(q, torch, dl, xd, rd, T, True)
            got, out = _run(q, torch, dl, xd, rd, T, False)
            for key in ref:
                assert np.array_equal(np.asarray(got[key]), np.asarray(ref[key])), (name, T, key)
            a = moegen.bf16_to_f32(out).astype(np.float64)
            b = moegen.bf16_to_f32(out_ref).astype(np.float64)
            # one bf16 step of the value, plus the fp32 order difference of
            # terms up to the row's largest magnitude (results near zero)
            bound = np.abs(b) * 2.0 ** -7 + np.abs(b).max(axis=1, keepdims=True) * 2.0 ** -20
            assert (np.abs(a - b) <= bound).all(), (name, T, float(np.abs(a - b).max()))
            g = {"logits": got["logits"].view(np.float32), "idx": got["idx"],
                 "w": got["w"].view(np.float32)}
            _, idx, wt = check_route(g, L, x)
            o_out = oracle.ffn_combine(L, x, idx, wt, res)
            check_out(out, o_out)
