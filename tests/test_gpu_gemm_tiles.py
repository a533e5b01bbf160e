"""GPU parity of the persistent grouped GEMM when its workgroups walk several
tiles each.  The persistent launch has two workgroups per CU; a workgroup
takes more than one tile only when a launch has more logical tiles (row block
x column tile) than workgroups, and only then do the hand-offs between tiles
run: the next tile's record and row table read during the last K step, the
rotation of the three row-table slots, the early switch of the weight
column base and the next tile's step 0 loaded by the current tile.  The
shape below gives both GEMMs about 1,100-2,200 logical tiles (4 or 5 per
workgroup) and 4 K steps each, over 64 experts of about 1,024 rows with a
ragged last row block each; every expert output is compared with the oracle,
for each down-projection format and both output types."""
import numpy as np
import pytest

import moegen
import oracle
from parity_util import check_buckets, check_route, check_y_rows, oracle_y, run_gpu

pytestmark = pytest.mark.gpu

_oracle_cache = {}


def _layer(fmt_down):
    w = moegen.Workload(name="tiles", E=64, k=8, H=512, I=512, T=8192, fmt_down=fmt_down)
    return w, moegen.make_layer(w)


@pytest.mark.parametrize("fmt_down", [moegen.FMT_NVFP4, moegen.FMT_Q6K, moegen.FMT_Q8_0,
                                      moegen.FMT_IQ3G, moegen.FMT_IQ1G])
@pytest.mark.parametrize("y_dtype", [0, 1])
def test_grouped_gemm_multi_tile_every_assignment(fmt_down, y_dtype):
    w, L = _layer(fmt_down)
    x = moegen.make_tokens(w, w.T, step=7)
    print("tiles fmt_down", fmt_down, "y_dtype", y_dtype, flush=True)
    g = run_gpu(L, x, y_dtype=y_dtype, ffn_mode=2)
    logits, idx, wt = check_route(g, L, x)
    ob = check_buckets(g["buckets"], idx, L.E)
    counts = ob["counts"].astype(np.int64)
    blocks = int(((counts + 127) // 128).sum())
    # more logical tiles than the 512 persistent workgroups of a 256-CU part,
    # in both GEMMs, and at least 4 K steps in each
    assert blocks * (w.I // 128) > 1024 and blocks * (w.H // 256) > 1024, blocks
    assert w.H // 128 >= 4 and w.I // 128 >= 4
    assert (counts % 128 != 0).sum() >= 32  # ragged last blocks
    if fmt_down not in _oracle_cache:
        _oracle_cache[fmt_down] = oracle_y(L, x, idx)
    oy = _oracle_cache[fmt_down]               # assignment order
    gy = g["y"][ob["asg_pos"]]                  # sorted order -> assignment order
    r, worst = check_y_rows(gy, oy)
    print(f"  rows {gy.shape[0]} rel L2 {r:.2e} worst row {worst:.2e}", flush=True)
