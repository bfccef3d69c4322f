"""Row-tile boundaries of the grouped GEMM, against the CPU oracle on every
output row.  Top-1 routing written on the host sets each expert's row count
directly: counts at and around the 32-row MFMA groups and the 128-row (Q8_0)
and 160-row (Q4_0) tiles, experts with no rows, and one expert with several
tiles.  The shared expert (Q4_0) runs all 1891 rows as 160-row tiles with a
131-row last tile.  The schedule's XCD ranges split this list by work, so
range boundaries fall inside the larger experts' tiles."""

import numpy as np
import pytest
import torch

import moegen
from moegen.configs import LayerConfig
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen
COUNTS = [1, 0, 31, 32, 33, 127, 128, 0, 129, 159, 160, 161, 289, 320, 0, 321]
TILES = LayerConfig(9, "tiles: H=512 F=512 E=16 k=1 shared q4_0", 512, len(COUNTS), 1, 512,
                    C.Q4_0, C.BF16, C.BF16, C.SOFTMAX, 0.02, shared_ffn=256, shared_q=C.Q4_0)


def _ids():
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(COUNTS)])
    np.random.default_rng(9).shuffle(ids)   # an expert's rows gather scattered tokens
    return ids[:, None]


@pytest.mark.parametrize("qtype", [C.Q4_0, C.Q8_0, C.Q4_K])
def test_tile_boundaries(ref, qtype):
    cfg = TILES
    ids = _ids()
    T = ids.shape[0]
    print(f"tile rows {qtype} T={T} counts={COUNTS}", flush=True)
    dl = G.layer(cfg, qtype=qtype)
    desc = G.desc_of(cfg, path="gemm", qtype=qtype)
    x = moegen.make_x(cfg, T, device=G.DEV)
    w = np.ones((T, 1), np.float32)
    ws = G.workspace(desc, T)
    off, sp, inv = G.permute(desc, cfg, torch.from_numpy(ids).to(G.DEV), ws)
    out = G.forward(desc, cfg, dl, x, torch.from_numpy(w).to(G.DEV), off, sp, inv, ws)
    torch.cuda.synchronize()
    assert fw.fw_moe_read_status(ws) == 0
    assert np.array_equal(np.diff(off.cpu().numpy()), COUNTS)
    want = G.oracle_forward(ref, cfg, dl, moegen.as_numpy_bits(x), ids, w)
    G.check_out(out.cpu().numpy(), want)
