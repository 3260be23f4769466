"""Write-disjointness of scatters on the GPU (hp_validate_writes and the
HP_FLAG_DISJOINT form of the scatters) against the oracle: the status and the
smallest clashing sequence, and that a rejected scatter writes nothing
([Hurray] Prefix Sharing: slices may name the same page; Partial trailing
page: the zeroed tail slots are writes too)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, assert_bits_equal, host_bits, idx_tensor, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def want(w, zero_tail):
    first = oracle.disjoint_writes(num_pages=w.num_pages, page_size=w.page_size,
                                   block_table=w.block_table, seq_ptr=w.seq_ptr,
                                   seq_lens=w.seq_lens, seq_start=w.seq_start,
                                   zero_tail=zero_tail)
    return ("HP_OK", 0) if first is None else ("HP_ERR_WRITE_ALIAS", first)


def small(seed, **kw):
    args = dict(max_seqs=8, max_len=60, heads=(1, 2), dims=(4, 8), dtypes=("f16",),
                alias=True, with_start=seed % 2 == 0)
    args.update(kw)
    return workloads.random_small(seed, **args)


def test_validate_writes_matches_oracle(hp):
    """300 small descriptors with aliased slices (30 % of entries repeat an
    earlier page), start offsets on half of them, both tail modes: the code
    and the smallest clashing sequence equal the oracle's."""
    clash = clean = 0
    for seed in range(2000, 2300):
        w = small(seed)
        d = OnDevice(w)
        for zt in (False, True):
            say("validate_writes", seed, zt, w.describe())
            got = hp.validate_writes(d.desc, w.total_tokens, d.ss, zero_tail=zt)
            assert got == want(w, zt), (seed, zt)
            clash += got[0] == "HP_ERR_WRITE_ALIAS"
            clean += got[0] == "HP_OK"
    assert clash > 60 and clean > 60, (clash, clean)


def test_validate_writes_reports_descriptor_errors_first(hp):
    """A descriptor that fails validation gets the validator's code, not a
    clash (the slot check only runs on a valid descriptor)."""
    w = small(2301, num_seqs=4, max_len=30, with_start=False)
    bt = w.block_table.copy()
    bt[0] = w.num_pages + 5
    bad = dataclasses.replace(w, block_table=bt)
    d = OnDevice(bad)
    say("validate_writes bad page", bad.describe())
    assert hp.validate_writes(d.desc, bad.total_tokens) == ("HP_ERR_PAGE_RANGE", 0)


def _scatter_case(hp, w, zero_tail, fn):
    """Runs fn(desc tensors) on a pool with known contents; returns the pool
    bits before and after and the status name (HP_OK or the error)."""
    d = OnDevice(w)
    before = host_bits(d.pool)
    try:
        fn(d)
        name = "HP_OK"
    except hp.HpError as e:
        name = e.name
    torch.cuda.synchronize()
    return d, before, host_bits(d.pool), name


def test_disjoint_scatter_writes_nothing_on_a_clash(hp):
    """Scatters with the disjoint check: on a clash HP_ERR_WRITE_ALIAS and the
    pool keeps every byte; otherwise the pool equals the oracle's scatter."""
    seen = set()
    for seed in range(2400, 2480):
        w = small(seed)
        for zt in (False, True):
            exp = want(w, zt)[0]
            say("disjoint scatter", seed, zt, exp, w.describe())
            src = w.make_src(DEV)
            d, before, after, name = _scatter_case(
                hp, w, zt, lambda d: hp.scatter(d.desc, src, d.ss, zero_tail=zt, disjoint=True))
            assert name == exp, (seed, zt)
            if exp == "HP_OK":
                ref = oracle.scatter(before, host_bits(src), zero_tail=zt,
                                     **d.oracle_kw(with_start=w.seq_start is not None))
                assert_bits_equal(after, ref, f"disjoint scatter {seed}")
            else:
                assert_bits_equal(after, before, f"rejected scatter {seed}")
            seen.add(exp)
    assert seen == {"HP_OK", "HP_ERR_WRITE_ALIAS"}


def test_disjoint_quantize_on_scatter_and_batch(hp):
    """The same check in quantize-on-scatter (codes and scales untouched on a
    clash; on a clean call the result equals the checked call without the
    slot check) and in the batched scatter (no member pool touched)."""
    seen = set()
    for seed in range(2500, 2540):
        w = small(seed, dtypes=("i8",))
        zt = seed % 3 == 0
        exp = want(w, zt)[0]
        say("disjoint quantize-on-scatter", seed, zt, exp, w.describe())
        src = torch.randn((w.total_tokens, w.num_heads, w.head_dim), device=DEV,
                          generator=torch.Generator(device=DEV).manual_seed(seed)).half()
        d = OnDevice(w)
        pool0, sc0 = d.pool.clone(), d.scales.clone()
        try:
            hp.scatter_quant(d.desc, src, d.ss, zero_tail=zt, disjoint=True)
            name = "HP_OK"
        except hp.HpError as e:
            name = e.name
        torch.cuda.synchronize()
        assert name == exp, (seed, zt)
        if exp == "HP_OK":
            ref = OnDevice(w, pool=pool0.clone())
            ref.scales.copy_(sc0)
            hp.scatter_quant(ref.desc, src, ref.ss, zero_tail=zt, checked=True)
            torch.cuda.synchronize()
            assert np.array_equal(host_bits(d.pool), host_bits(ref.pool))
            assert np.array_equal(host_bits(d.scales), host_bits(ref.scales))
        else:
            assert np.array_equal(host_bits(d.pool), host_bits(pool0))
            assert np.array_equal(host_bits(d.scales), host_bits(sc0))
        seen.add(exp)
    assert seen == {"HP_OK", "HP_ERR_WRITE_ALIAS"}
    # batched: three pools sharing the table
    for seed in range(2600, 2640):
        w = small(seed, with_start=True)
        exp = want(w, True)[0]
        if exp == "HP_OK":
            continue
        say("disjoint batched scatter", seed, w.describe())
        d = OnDevice(w)
        pools = [w.make_pool(DEV) for _ in range(3)]
        copies = [p.clone() for p in pools]
        srcs = [w.make_src(DEV) for _ in range(3)]
        with pytest.raises(hp.HpError) as e:
            hp.scatter_batch(d.desc, pools, srcs, d.ss, zero_tail=True, disjoint=True)
        torch.cuda.synchronize()
        assert e.value.name == "HP_ERR_WRITE_ALIAS"
        # bit patterns (the seeded pools may hold NaNs, which never compare equal)
        assert all(np.array_equal(host_bits(p), host_bits(c)) for p, c in zip(pools, copies))
        return
    pytest.fail("no clashing batch among the seeds")


def test_disjoint_full_size_decode_and_quant(hp):
    """The decode batch (64 sequences over 12,000 unique pages) is clean;
    after pointing sequence 40's first page at sequence 10's the smallest
    clashing sequence is 10. The 1.65M-token int8 pool with its uint64 table
    (200,000 pages) against the oracle too."""
    w = workloads.decode()
    say("disjoint decode full", w.describe())
    d = OnDevice(w)
    assert hp.validate_writes(d.desc, w.total_tokens) == want(w, False) == ("HP_OK", 0)
    assert hp.validate_writes(d.desc, w.total_tokens, zero_tail=True) == want(w, True)
    bt = w.block_table.copy()
    bt[int(w.seq_ptr[40])] = bt[int(w.seq_ptr[10])]
    w2 = dataclasses.replace(w, block_table=bt)
    d.bt.copy_(idx_tensor(bt.astype(w.index_dtype), DEV))
    torch.cuda.synchronize()
    assert want(w2, False) == ("HP_ERR_WRITE_ALIAS", 10)
    assert hp.validate_writes(d.desc, w.total_tokens) == ("HP_ERR_WRITE_ALIAS", 10)
    del d
    torch.cuda.empty_cache()
    q = workloads.quant()
    say("disjoint quant full", q.describe())
    dq = OnDevice(q)
    for zt in (False, True):
        assert hp.validate_writes(dq.desc, q.total_tokens, zero_tail=zt) == want(q, zt)
    del dq
    torch.cuda.empty_cache()


def test_disjoint_empty_batch(hp):
    w = workloads.Workload("empty", "f16", 16, 2, 8, 4, np.uint32, np.zeros(0, np.uint32),
                           np.zeros(1, np.uint32), np.zeros(0, np.uint32), seed=1)
    d = OnDevice(w)
    say("disjoint empty batch")
    assert hp.validate_writes(d.desc, 0) == ("HP_OK", 0)
