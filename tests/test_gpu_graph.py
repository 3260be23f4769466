"""The unchecked entry points can be captured in a HIP graph: gather,
scatter, dequant-gather and decode attention are recorded once and replayed
several times, with eager work and synchronisations between the replays.
Every replay must reproduce the eager results bit for bit (the same kernels
on the same inputs)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_util import OnDevice, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def test_capture_and_replay(hp):
    w = workloads.random_small(1600, max_seqs=24, max_len=400, page_sizes=(16,), heads=(4,),
                               dims=(64,), dtypes=("bf16",), alias=False)
    say("graph capture", w.describe())
    d = OnDevice(w)
    T = w.total_tokens
    v_pool = dataclasses.replace(w, seed=w.seed + 1).make_pool(DEV)
    wq = dataclasses.replace(w, dtype="i8", values="int8", with_scales=True, seed=w.seed + 2)
    qpool, scales = wq.make_pool(DEV), wq.make_scales(DEV)
    qdesc = hp.Descriptor(qpool, d.bt, d.sp, d.sl, scales=scales)
    g = torch.Generator(device=DEV).manual_seed(1601)
    q = torch.randn((w.num_seqs, 8, 64), generator=g, device=DEV).to(torch.bfloat16)
    src = w.make_src(DEV)
    scatter_pool = torch.zeros_like(d.pool)
    sdesc = hp.Descriptor(scatter_pool, d.bt, d.sp, d.sl)
    ws = torch.empty(max(hp.attention_workspace_bytes(d.desc, T, 8), 256), dtype=torch.uint8,
                     device=DEV)

    gout = torch.empty((T, 4, 64), dtype=torch.bfloat16, device=DEV)
    qout = torch.empty((T, 4, 64), dtype=torch.bfloat16, device=DEV)
    aout = torch.empty((w.num_seqs, 8, 64), dtype=torch.float32, device=DEV)

    def work(stream=None):
        hp.gather(d.desc, gout, stream=stream)
        hp.scatter(sdesc, src, stream=stream)
        hp.gather_dequant(qdesc, qout, stream=stream)
        hp.paged_attention(d.desc, v_pool, q, aout, total_tokens=T, workspace=ws, stream=stream)

    work()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (gout, scatter_pool, qout, aout)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        # the graph records on `side`; every call names that stream
        for t in (gout, qout, aout):
            t.zero_()
        scatter_pool.zero_()
        with torch.cuda.graph(graph, stream=side):
            work(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (gout, qout, aout):
            t.fill_(float("nan"))
        scatter_pool.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("gather", "scatter", "dequant", "attention"),
                                   (gout, scatter_pool, qout, aout), eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), (rep, name)
        # eager work between the replays
        hp.gather(d.desc, gout)
        torch.cuda.synchronize()
    graph.reset()
