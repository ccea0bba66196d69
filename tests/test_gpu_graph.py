"""The hot path captured in a HIP graph: every replay matches the eager
result bit for bit, with eager work and synchronisations between replays
(the library launches only kernels on the caller's stream, no memsets)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_253_amd as pk
from workloads import WORKLOADS, make_batch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx,p", [(2, -1), (2, 512), (5, 512), (1, 0)])
def test_graph_replays_match_eager(idx, p):
    w = WORKLOADS[idx]
    lens = None if idx == 1 else (np.array([700, 1500, 3000, 4096]) if idx == 2 else np.array([4000, 2500]))
    batch = make_batch(w, device="cuda", lens=lens)
    dev = batch.k_pool.device
    bt = torch.from_numpy(batch.block_tables).to(dev)
    cl = torch.from_numpy(batch.context_lens).to(dev)
    slots = torch.from_numpy(batch.slot_mapping).to(dev)
    out = torch.empty_like(batch.q)
    s, hq, d = batch.q.shape
    ws = None
    if p:
        ws = torch.zeros(pk.workspace_size(s, hq, w.num_kv_heads, d, batch.max_context_len, p),
                         dtype=torch.uint8, device=dev)

    def step():
        pk.kv_cache_write(batch.k_new, batch.v_new, batch.k_pool, batch.v_pool, slots,
                          batch.k_scale, batch.v_scale)
        pk.decode(batch.q, batch.k_pool, batch.v_pool, bt, cl, batch.max_context_len,
                  batch.scale, batch.k_scale, batch.v_scale, p, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        out.fill_(float("nan"))        # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
