"""The ABI keeps no state between calls: two host threads, each with its own
stream, workspace and buffers, run fw_moe_layer at the same time and get the
serial results bit for bit (ctypes releases the GIL inside each call, so the
library's host code runs concurrently too)."""

import threading

import pytest
import torch

import moegen
from sparse_moe_block_amd import fwmoe as fw
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

C = moegen


def _buffers(cfg, desc, T):
    E, k, P = cfg.n_experts, cfg.top_k, T * cfg.top_k
    return dict(logits=torch.empty(T, E, device=G.DEV),
                ids=torch.empty(T, k, dtype=torch.int32, device=G.DEV),
                w=torch.empty(T, k, device=G.DEV),
                off=torch.empty(E + 1, dtype=torch.int32, device=G.DEV),
                sp=torch.empty(P, dtype=torch.int32, device=G.DEV),
                inv=torch.empty(P, dtype=torch.int32, device=G.DEV),
                out=torch.empty(T, cfg.hidden, device=G.DEV),
                ws=G.workspace(desc, T))


def _layer(desc, T, x, L, b, stream):
    fw.fw_moe_layer(desc, T, x, L.router, L.bias, L.w_gate, L.w_up, L.w_down, L.s_gate,
                    L.s_up, L.s_down, b["logits"], b["ids"], b["w"], b["off"], b["sp"],
                    b["inv"], b["out"], b["ws"], stream=stream)


@pytest.mark.parametrize("T,path", [(16, "auto"), (300, "auto"), (16, "gemm")])
def test_two_threads_match_serial(T, path):
    print(f"two threads qwen3 T={T} {path}", flush=True)
    cfg = C.QWEN3_DECODE
    dl = G.layer(cfg)
    desc = G.desc_of(cfg, path=path)
    xs = [moegen.make_x(cfg, T, device=G.DEV, variant=v) for v in (1, 2)]
    # serial references
    refs = []
    for x in xs:
        b = _buffers(cfg, desc, T)
        _layer(desc, T, x, dl.L, b, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert fw.fw_moe_read_status(b["ws"]) == 0
        refs.append(b["out"].clone())
    streams = [torch.cuda.Stream() for _ in xs]
    bufs = [_buffers(cfg, desc, T) for _ in xs]
    outs = [[] for _ in xs]
    errors = []
    start = threading.Barrier(len(xs))

    def worker(i):
        try:
            start.wait()
            for _ in range(20):
                _layer(desc, T, xs[i], dl.L, bufs[i], streams[i])
                o = torch.empty_like(bufs[i]["out"])
                with torch.cuda.stream(streams[i]):
                    o.copy_(bufs[i]["out"])
                outs[i].append(o)
        except Exception as e:   # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(xs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(xs)):
        assert fw.fw_moe_read_status(bufs[i]["ws"]) == 0
        for o in outs[i]:
            assert torch.equal(o, refs[i])
