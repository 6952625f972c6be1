"""The wide configuration's split down-phase tail (hybrid Stream-K over the wide
grid): at loads whose down phase has one or more full rounds and a last round of
at most half the grid, each tail tile is computed in pieces by several
workgroups and a fix-up launch adds them.  The split rule and the tile order are
evaluated from their specification (tests/spec.py) on the oracle's alignment, so
each case is known to split; Y is compared with the oracle on tokens whose rows
lie in split tiles, plus a random sample."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_helpers as G
from tests import spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


@pytest.mark.parametrize("shape,B,alpha,P_expected", [
    ("mixtral", 1536, 1.0, 16), ("mixtral", 2048, 0.1, 8), ("mixtral", 2048, 1.0, 4),
    ("mixtral", 2304, 1.0, 2), ("qwen3", 1024, 1.0, 3), ("qwen3", 4096, 3.0, 3),
])
def test_wide_split_tail(shape, B, alpha, P_expected):
    grid = min(G.num_cus(), 512)
    if grid != 256:
        pytest.skip("the expected piece counts assume a 256-CU GPU")
    G.say(f"wide split {shape} B={B} alpha={alpha}")
    wdev, whost = G.weights(shape)
    layer = synth.make_layer(shape, B, alpha, 0, weights=whost)
    sh = layer.shape
    ids, w = oracle.route_topk(layer.logits, sh.top_k)
    bm = spec.MENU[spec.WIDE][0]
    ss, be, nb, _ = oracle.align(ids, layer.expert_begin, sh.local_experts, bm)
    ncol = -(-sh.hidden // spec.MENU[spec.WIDE][2])
    total = nb * ncol
    P = spec.wide_pieces(total, grid, sh.inter // 32)
    assert P == P_expected, (nb, total, P)
    # tokens with a slot in the row-blocks of split tiles
    F = total // grid
    split_rbs = sorted({spec.expert_major_tile(t, be, ncol)[0] for t in range(F * grid, total)})
    rng = np.random.default_rng([B, 5])
    picked = set()
    for rb in split_rbs:
        # one token in each 64-row quarter of the row-block (each quarter is added
        # by its own wave and fix-up workgroup)
        for q in range(bm // 64):
            rows = ss[rb * bm + q * 64:rb * bm + (q + 1) * 64]
            rows = rows[rows >= 0]
            if len(rows):
                picked.add(int(rng.choice(rows)) // sh.top_k)
    toks = np.array(sorted(picked | set(rng.choice(B, 12, replace=False).tolist())), dtype=np.int32)
    out = G.fetch(G.run(layer, variant=spec.WIDE, wdev=wdev))
    G.check_routing(layer, out)
    G.check_align(layer, out, ids)
    err, _ = G.check_y(layer, out, ids, w, toks)
    G.say(f"  P={P}, {len(split_rbs)} split row-blocks, rel err {err:.3g} on {len(toks)} tokens")
