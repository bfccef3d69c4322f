"""GPU parity of fw_moe_permute on random id tables: the one-workgroup sort (up
to 2048 pairs), the multi-workgroup sort with the scan folded into the scatter
(up to 64 chunks of 1024 pairs) and with a separate scan kernel, with ragged
last chunks, extreme skew, every expert count up to 512 and out-of-range ids."""

import numpy as np
import pytest
import torch

from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# (E, k, T, distribution, fraction of out-of-range ids)
CASES = [
    (64, 4, 100, "uniform", 0.05),    # one workgroup, bad ids
    (64, 4, 512, "uniform", 0.0),     # P = 2048: the one-workgroup limit
    (8, 2, 1025, "uniform", 0.0),     # P = 2050: three chunks, the last of 2 pairs
    (100, 5, 777, "uniform", 0.0),    # E not a multiple of 64, ragged last chunk
    (512, 16, 300, "uniform", 0.01),  # E = 512, k = 16, bad ids
    (128, 8, 2048, "one", 0.0),       # every pair to one expert
    (256, 8, 4096, "zipf", 0.0),      # skewed, 32 chunks
    (128, 8, 3000, "zipf", 0.02),     # skewed, ragged, bad ids
    (64, 8, 9000, "zipf", 0.001),     # 71 chunks: the separate per-expert scan
]


def _ids(E, k, T, dist, bad, seed):
    rng = np.random.default_rng(seed)
    if dist == "one":
        ids = np.full((T, k), 3, np.int64)   # every slot of every token: expert 3
    elif dist == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        ids = rng.choice(E, size=(T, k), p=p / p.sum())
    else:
        ids = rng.integers(0, E, (T, k))
    if bad > 0:
        m = rng.random((T, k)) < bad
        ids[m] = rng.choice(np.array([-1, E, E + 7, 2**31 - 1]), size=int(m.sum()))
    return ids.astype(np.int32)


def _expected(ref, ids, E):
    """The oracle's stable sort with every out-of-range id mapped to an extra
    expert E: its first E + 1 offsets and first offsets[E] sorted entries are
    the valid pairs' result; the rest of the list is -1, and so is inv_pos of
    an out-of-range pair."""
    bad = (ids < 0) | (ids >= E)
    off, sp, inv = ref.permute(np.where(bad, E, ids).astype(np.int32), E + 1)
    n = off[E]
    sp = sp.copy()
    sp[n:] = -1
    inv = inv.copy()
    inv[bad.reshape(-1)] = -1
    return off[:E + 1], sp, inv, bool(bad.any())


@pytest.mark.parametrize("E,k,T,dist,bad", CASES,
                         ids=[f"E{c[0]}-k{c[1]}-T{c[2]}-{c[3]}-bad{c[4]}" for c in CASES])
def test_permute_random(ref, E, k, T, dist, bad):
    print(f"permute E={E} k={k} T={T} {dist} bad={bad}", flush=True)
    ids = _ids(E, k, T, dist, bad, seed=E * 131 + T)
    desc = fw.make_desc(256, E, k, 256)
    ws = G.workspace(desc, T)
    off, sp, inv = G.permute(desc, _Cfg(E, k), torch.from_numpy(ids).to(G.DEV), ws)
    roff, rsp, rinv, has_bad = _expected(ref, ids, E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(inv.cpu().numpy(), rinv)
    st = fw.fw_moe_read_status(ws)
    assert st == (fw.FW_STATUS_BAD_EXPERT_ID if has_bad else 0)


def test_permute_reuses_workspace(ref):
    """Two large sorts in a row on one workspace (the per-chunk counts of the
    first must not leak into the second), then a small one."""
    E, k = 128, 8
    desc = fw.make_desc(256, E, k, 256)
    ws = G.workspace(desc, 4096)
    for T, seed in [(4096, 1), (2500, 2), (16, 3)]:
        ids = _ids(E, k, T, "zipf", 0.0, seed)
        off, sp, inv = G.permute(desc, _Cfg(E, k), torch.from_numpy(ids).to(G.DEV), ws)
        roff, rsp, rinv, _ = _expected(ref, ids, E)
        assert np.array_equal(off.cpu().numpy(), roff)
        assert np.array_equal(sp.cpu().numpy(), rsp)
        assert np.array_equal(inv.cpu().numpy(), rinv)
    assert fw.fw_moe_read_status(ws) == 0


def test_permute_large_needs_workspace():
    """Above 2048 pairs the sort keeps per-chunk counts in the workspace: a
    status-word-only workspace is refused before anything is launched."""
    E, k, T = 64, 8, 512
    desc = fw.make_desc(256, E, k, 256)
    ws = torch.zeros(256, dtype=torch.uint8, device=G.DEV)
    ids = torch.zeros((T, k), dtype=torch.int32, device=G.DEV)
    off = torch.zeros(E + 1, dtype=torch.int32, device=G.DEV)
    sp = torch.zeros(T * k, dtype=torch.int32, device=G.DEV)
    inv = torch.zeros(T * k, dtype=torch.int32, device=G.DEV)
    with pytest.raises(fw.FwMoeError) as e:
        fw.fw_moe_permute(desc, T, ids, off, sp, inv, ws)
    assert e.value.code == fw.FW_EWORKSPACE


class _Cfg:
    def __init__(self, E, k):
        self.n_experts, self.top_k = E, k
