"""Row-tile boundaries of the grouped GEMM, against the CPU oracle on every
output row.  Top-1 routing written on the host sets each expert's row count
directly: counts at and around the 32-row MFMA groups and the 128-row (Q8_0)
and 160-row (Q4_0) tiles, experts with no rows, and one expert with several
tiles.  The shared expert runs all 1891 rows as 160-row (Q4_0, fp16
activations; MXFP4, MXFP8 activations) or 128-row tiles, the last one partial.
The same row counts go through the two activation-quantising modes: the
block-scaled GEMM (160-row tiles, five groups split three and two over the
row halves) and the int8 GEMM (128-row tiles).  The schedule's XCD ranges
split the tile list by work or by count, so range boundaries fall inside the
larger experts' tiles; the ranges the schedule writes into the workspace
header are checked against the tile count and the launch's room per XCD."""

import numpy as np
import pytest
import torch

import moegen
from moegen.configs import LayerConfig
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G
from tests.test_gpu_int8 import check_int8, h_step_max
from tests.test_gpu_mx8 import check_mx8

pytestmark = pytest.mark.gpu

C = moegen
COUNTS = [1, 0, 31, 32, 33, 127, 128, 0, 129, 159, 160, 161, 289, 320, 0, 321]
TILES = LayerConfig(9, "tiles: H=512 F=512 E=16 k=1 shared q4_0", 512, len(COUNTS), 1, 512,
                    C.Q4_0, C.BF16, C.BF16, C.SOFTMAX, 0.02, shared_ffn=256, shared_q=C.Q4_0)


MODES = {"mxfp8": TILES.with_(expert_q=C.MXFP4, shared_q=C.MXFP4, act_quant="mxfp8"),
         "int8": TILES.with_(act_quant="int8")}


# tile rows of each kernel (the fp16 GEMM by expert format)
TILE_ROWS = {C.Q4_0: 160, C.Q8_0: 128, C.Q4_K: 128, "mxfp8": 160, "int8": 128}


def _check_xcd_ranges(ws, P, E, tile_rows):
    """Header: status, active experts, tiles, then the 9 XCD range bounds."""
    hdr = ws[:48].cpu().numpy().view(np.int32)
    n_tiles, first = int(hdr[2]), hdr[3:12]
    want_tiles = sum((n + tile_rows - 1) // tile_rows for n in COUNTS)
    assert n_tiles == want_tiles
    max_tiles = (P + 1) // 2 + E                 # the workspace's tile list
    cap = (min((P + tile_rows - 1) // tile_rows + E, max_tiles) + 7) // 8
    assert first[0] == 0 and first[8] == n_tiles
    assert np.all(np.diff(first) >= 0) and np.all(np.diff(first) <= cap), first


def _ids():
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(COUNTS)])
    np.random.default_rng(9).shuffle(ids)   # an expert's rows gather scattered tokens
    return ids[:, None]


def _run(ref, cfg, qtype=None, tile_rows=None):
    ids = _ids()
    T = ids.shape[0]
    print(f"tile rows {qtype or cfg.expert_q} act_quant={cfg.act_quant} T={T} "
          f"counts={COUNTS}", flush=True)
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
    _check_xcd_ranges(ws, T, cfg.n_experts, tile_rows)
    want = G.oracle_forward(ref, cfg, dl, moegen.as_numpy_bits(x), ids, w)
    return out.cpu().numpy(), want, desc, ws, T


@pytest.mark.parametrize("qtype", [C.Q4_0, C.Q8_0, C.Q4_K])
def test_tile_boundaries(ref, qtype):
    got, want, _, _, _ = _run(ref, TILES, qtype, TILE_ROWS[qtype])
    G.check_out(got, want)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_tile_boundaries_quantised_activations(ref, mode):
    cfg = MODES[mode]
    got, want, desc, ws, T = _run(ref, cfg, tile_rows=TILE_ROWS[mode])
    if mode == "mxfp8":
        check_mx8(got, want)
    else:
        check_int8(got, want, h_step_max(desc, cfg, ws, T))
