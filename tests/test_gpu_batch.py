"""GPU parity of the batched calls: several pools moved through one shared
block table in one call. Member i must equal the oracle on pool i (and the
single call on pool i), bit for bit; dequant with tolerance 0."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, assert_bits_equal, bf16_bits_equal, host_bits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def members(w, count):
    """`count` workloads with the same table and different pool contents."""
    return [dataclasses.replace(w, seed=w.seed * 1000 + 17 + i) for i in range(count)]


def _kw(w, with_start=False):
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    if with_start:
        kw["seq_start"] = w.seq_start
    return kw


@pytest.mark.parametrize("streaming", [False, True])
@pytest.mark.parametrize("seed,count", [(7, 1), (8, 5), (9, 33), (10, 40)])
def test_gather_batch(hp, seed, count, streaming):
    w = workloads.random_small(600 + seed, max_seqs=24, max_len=400,
                               page_sizes=(3, 16), heads=(2, 8), dims=(16, 128))
    say("gather batch", seed, count, streaming, w.describe())
    d = OnDevice(w)
    ms = members(w, count)
    pools = [m.make_pool(DEV) for m in ms]
    outs = [d.empty_out() for _ in ms]
    hp.gather_batch(d.desc, pools, outs, streaming=streaming)
    torch.cuda.synchronize()
    for i, (m, pool, out) in enumerate(zip(ms, pools, outs)):
        assert_bits_equal(host_bits(out), oracle.gather(host_bits(pool), **_kw(w)),
                          f"member {i}")
    single = d.empty_out()
    hp.gather(hp.Descriptor(pools[-1], d.bt, d.sp, d.sl), single, streaming=streaming)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(outs[-1]), host_bits(single), "batch == single")


def test_gather_batch_plan_path(hp):
    """More sequences than the LDS table holds: the plan kernels run once and
    every member's launch reuses them (34 members = two launches)."""
    rng = np.random.default_rng(12)
    w = None
    while w is None or w.num_seqs <= 4096:
        w = workloads.random_small(int(rng.integers(1 << 30)), max_seqs=7000, max_len=12,
                                   page_sizes=(4,), heads=(1,), dims=(16,), dtypes=("f16",))
    say("gather batch plan path", w.describe())
    d = OnDevice(w)
    ms = members(w, 34)
    pools = [m.make_pool(DEV) for m in ms]
    outs = [d.empty_out() for _ in ms]
    hp.gather_batch(d.desc, pools, outs, checked=True)
    torch.cuda.synchronize()
    for i in (0, 1, 31, 32, 33):
        assert_bits_equal(host_bits(outs[i]), oracle.gather(host_bits(pools[i]), **_kw(w)),
                          f"member {i}")


@pytest.mark.parametrize("zero_tail", [False, True])
@pytest.mark.parametrize("seed,count", [(1, 3), (2, 6), (3, 35)])
def test_scatter_batch(hp, seed, count, zero_tail):
    w = workloads.random_small(700 + seed, max_seqs=24, max_len=300, page_sizes=(4, 16),
                               heads=(2, 8), dims=(16, 128), alias=False, with_start=True)
    say("scatter batch", seed, count, zero_tail, w.describe())
    d = OnDevice(w)
    ms = members(w, count)
    pools = [m.make_pool(DEV) for m in ms]
    srcs = [m.make_src(DEV) for m in ms]
    want = [oracle.scatter(host_bits(p), host_bits(s), zero_tail=zero_tail,
                           **_kw(w, with_start=True)) for p, s in zip(pools, srcs)]
    hp.scatter_batch(d.desc, pools, srcs, d.ss, zero_tail=zero_tail, checked=True)
    torch.cuda.synchronize()
    for i, (pool, wt) in enumerate(zip(pools, want)):
        assert_bits_equal(host_bits(pool), wt, f"member {i}")


@pytest.mark.parametrize("seed,count", [(1, 2), (2, 4), (3, 33)])
def test_dequant_batch(hp, seed, count):
    w = workloads.random_small(800 + seed, max_seqs=20, max_len=300, page_sizes=(8, 16),
                               heads=(1, 8), dims=(16, 128), dtypes=("i8",))
    say("dequant batch", seed, count, w.describe())
    d = OnDevice(w)
    ms = members(w, count)
    pools = [m.make_pool(DEV) for m in ms]
    scales = [m.make_scales(DEV) for m in ms]
    outs = [d.empty_out(dtype=torch.bfloat16) for _ in ms]
    hp.gather_dequant_batch(d.desc, pools, scales, outs)
    torch.cuda.synchronize()
    for i, (pool, sc, out) in enumerate(zip(pools, scales, outs)):
        want = oracle.gather_dequant(host_bits(pool).view(np.int8), sc.cpu().numpy(), **_kw(w))
        bf16_bits_equal(host_bits(out), want, f"member {i}")
