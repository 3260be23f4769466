"""GPU tests of the enqueue-only checked form: hp_validate_async leaves its
verdict on the device and moves called with HP_FLAG_GATED read it there
([Hurray] Storage Invariants: a descriptor that violates the invariants is
rejected). A valid descriptor's gated moves equal the oracle bit for bit; a
rejected one's leave every output, pool slot, scale and zero point as it was,
and the verdict read back equals hp_validate's and the oracle's."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_bits_equal, bf16_bits_equal, fill_bits, host_bits, idx_tensor, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = {"valid": "HP_OK", "seq_ptr_first": "HP_ERR_SEQPTR_FIRST",
         "seq_ptr_last": "HP_ERR_SEQPTR_LAST", "seq_ptr_order": "HP_ERR_SEQPTR_ORDER",
         "page_range": "HP_ERR_PAGE_RANGE", "seq_len": "HP_ERR_SEQ_LEN",
         "total_tokens": "HP_ERR_TOTAL_TOKENS"}


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def corrupted(seed):
    """A valid descriptor without aliased pages (so that its scatter is
    defined), then 0..3 random corruptions of its table, offsets, counts or
    total. Returns the workload and the (possibly) corrupted arrays."""
    rng = np.random.default_rng(seed)
    w = workloads.random_small(6000 + seed, max_seqs=12, max_len=120, alias=False,
                               with_start=bool(seed % 2), dtypes=("f16", "bf16", "f32", "u8"))
    bt = w.block_table.astype(np.int64).tolist()
    sp = w.seq_ptr.astype(np.int64).tolist()
    sl = w.seq_lens.astype(np.int64).tolist()
    T = w.total_tokens
    for _ in range(int(rng.integers(0, 4))):
        kind = rng.integers(0, 5)
        if kind == 0 and sp:
            i = int(rng.integers(0, len(sp)))
            sp[i] = max(0, sp[i] + int(rng.integers(-2, 3)))
        elif kind == 1 and bt:
            bt[int(rng.integers(0, len(bt)))] = w.num_pages + int(rng.integers(0, 3))
        elif kind == 2 and sl:
            sl[int(rng.integers(0, len(sl)))] += int(rng.integers(1, 2 * w.page_size))
        elif kind == 3:
            T = max(0, T + int(rng.integers(-1, 2)))
        elif kind == 4 and bt:
            bt.pop()
    return w, bt, sp, sl, T


@pytest.mark.parametrize("seed", range(60))
def test_gated_moves(hp, seed):
    w, bt, sp, sl, T = corrupted(seed)
    dt = w.index_dtype
    say("gated moves", seed, w.describe(), "T", T)
    tbt = idx_tensor(np.array(bt, dtype=dt), DEV)
    tsp = idx_tensor(np.array(sp, dtype=dt), DEV)
    tsl = idx_tensor(np.array(sl, dtype=dt), DEV)
    ss = w.seq_start
    tss = idx_tensor(ss.astype(dt), DEV) if ss is not None else None
    pool = w.make_pool(DEV)
    desc = hp.Descriptor(pool, tbt, tsp, tsl)
    want = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages, page_size=w.page_size,
                           block_table=bt, seq_ptr=sp, seq_lens=sl, total_tokens=T,
                           seq_start=ss)
    ok = want[0] == "valid"
    ws = torch.full((max(hp.workspace_bytes(desc, T), 256),), 0x5A, dtype=torch.uint8,
                    device=DEV)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=np.array(bt, dtype=np.uint64), seq_ptr=np.array(sp, dtype=np.uint64),
              seq_lens=np.array(sl, dtype=np.uint64))

    # gather: the starts do not apply, so validate without them
    hp.validate_async(desc, T, workspace=ws)
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=pool.dtype, device=DEV)
    fill_bits(out, workloads.SENTINEL_BITS[out.element_size()])
    hp.gather(desc, out, workspace=ws, gated=True)
    torch.cuda.synchronize()
    want_g = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages,
                             page_size=w.page_size, block_table=bt, seq_ptr=sp, seq_lens=sl,
                             total_tokens=T)
    assert hp.validate_verdict(desc, T, ws) == (NAMES[want_g[0]], want_g[1])
    assert hp.validate(desc, T) == (NAMES[want_g[0]], want_g[1])
    if want_g[0] == "valid":
        assert_bits_equal(host_bits(out), oracle.gather(host_bits(pool), **kw), "gated gather")
    else:
        sentinel = workloads.SENTINEL_BITS[out.element_size()]
        assert np.all(host_bits(out) == sentinel), "rejected gather wrote its output"

    # scatter with the starts (and tail zeroing on odd seeds)
    zero_tail = bool(seed % 3 == 1)
    src = dataclasses.replace(w, seed=w.seed + 17).make_src(DEV)[:T] if T else \
        torch.empty((0, w.num_heads, w.head_dim), dtype=pool.dtype, device=DEV)
    if src.shape[0] != T:  # corrupted T above the workload's total: extra source rows
        src = torch.cat([src, src[:T - src.shape[0]]]) if src.shape[0] else src
    before = host_bits(pool)
    hp.validate_async(desc, T, tss, workspace=ws)
    if src.shape[0] == T:
        hp.scatter(desc, src, tss, zero_tail=zero_tail, workspace=ws, gated=True)
    torch.cuda.synchronize()
    assert hp.validate_verdict(desc, T, ws) == (NAMES[want[0]], want[1])
    if ok and src.shape[0] == T:
        want_pool = oracle.scatter(before, host_bits(src), seq_start=ss, zero_tail=zero_tail,
                                   **kw)
        assert_bits_equal(host_bits(pool), want_pool, "gated scatter")
    else:
        assert_bits_equal(host_bits(pool), before, "rejected scatter wrote the pool")


@pytest.mark.parametrize("seed", range(24))
def test_gated_dequant_and_quantize(hp, seed):
    """Dequant-gather and quantize-on-scatter through the gate: int8 pool
    with per-slot scales."""
    w, bt, sp, sl, T = corrupted(300 + seed)
    w = dataclasses.replace(w, dtype="i8", values="int8", with_scales=True)
    dt = w.index_dtype
    say("gated dequant / quantize", seed, w.describe(), "T", T)
    tbt = idx_tensor(np.array(bt, dtype=dt), DEV)
    tsp = idx_tensor(np.array(sp, dtype=dt), DEV)
    tsl = idx_tensor(np.array(sl, dtype=dt), DEV)
    ss = w.seq_start
    tss = idx_tensor(ss.astype(dt), DEV) if ss is not None else None
    pool, scales = w.make_pool(DEV), w.make_scales(DEV)
    desc = hp.Descriptor(pool, tbt, tsp, tsl, scales=scales)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=np.array(bt, dtype=np.uint64), seq_ptr=np.array(sp, dtype=np.uint64),
              seq_lens=np.array(sl, dtype=np.uint64))
    ws = torch.zeros(max(hp.workspace_bytes(desc, T), 256), dtype=torch.uint8, device=DEV)
    v_plain = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages,
                              page_size=w.page_size, block_table=bt, seq_ptr=sp, seq_lens=sl,
                              total_tokens=T)
    v_start = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages,
                              page_size=w.page_size, block_table=bt, seq_ptr=sp, seq_lens=sl,
                              total_tokens=T, seq_start=ss)

    hp.validate_async(desc, T, workspace=ws)
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
    fill_bits(out, workloads.SENTINEL_BITS[2])
    hp.gather_dequant(desc, out, workspace=ws, gated=True)
    torch.cuda.synchronize()
    assert hp.validate_verdict(desc, T, ws) == (NAMES[v_plain[0]], v_plain[1])
    if v_plain[0] == "valid":
        bf16_bits_equal(host_bits(out), oracle.gather_dequant(
            host_bits(pool).view(np.int8), scales.cpu().numpy(), **kw), "gated dequant")
    else:
        assert np.all(host_bits(out) == workloads.SENTINEL_BITS[2])

    g = torch.Generator(device=DEV).manual_seed(seed)
    src = torch.randn((T, w.num_heads, w.head_dim), generator=g, device=DEV).to(torch.float16)
    pool_before, sc_before = host_bits(pool).view(np.int8), scales.cpu().numpy()
    hp.validate_async(desc, T, tss, workspace=ws)
    hp.scatter_quant(desc, src, tss, zero_tail=True, workspace=ws, gated=True)
    torch.cuda.synchronize()
    assert hp.validate_verdict(desc, T, ws) == (NAMES[v_start[0]], v_start[1])
    if v_start[0] == "valid":
        want_pool, want_sc, _ = oracle.scatter_quant(pool_before, sc_before, host_bits(src), "f16",
                                                     seq_start=ss, zero_tail=True, **kw)
        assert np.array_equal(host_bits(pool).view(np.int8), want_pool), "gated quantize codes"
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_sc.view(np.uint32))
    else:
        assert np.array_equal(host_bits(pool).view(np.int8), pool_before)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), sc_before.view(np.uint32))


def test_gated_plan_path_and_batch(hp):
    """More sequences than the fused scan holds (plan arrays after the
    verdict words in the workspace) and a batched gather over three pools:
    accepted, then rejected after one page ID is pushed out of range."""
    w = workloads.random_small(6500, max_seqs=9000, max_len=30, page_sizes=(4, 16), heads=(2,),
                               dims=(64,), dtypes=("bf16",), num_seqs=5000, alias=False)
    say("gated plan path", w.describe())
    pools = [dataclasses.replace(w, seed=w.seed + i).make_pool(DEV) for i in range(3)]
    bt = w.block_table.copy()
    tbt = idx_tensor(bt, DEV)
    desc = hp.Descriptor(pools[0], tbt, idx_tensor(w.seq_ptr, DEV), idx_tensor(w.seq_lens, DEV))
    T = w.total_tokens
    ws = torch.empty(hp.workspace_bytes(desc, T), dtype=torch.uint8, device=DEV)
    outs = [torch.empty((T, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=DEV)
            for _ in pools]
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    hp.validate_async(desc, T, workspace=ws)
    hp.gather_batch(desc, pools, outs, workspace=ws, gated=True)
    torch.cuda.synchronize()
    assert hp.validate_verdict(desc, T, ws) == ("HP_OK", 0)
    for p, o in zip(pools, outs):
        assert_bits_equal(host_bits(o), oracle.gather(host_bits(p), **kw), "gated batch")
    # one page ID out of range: nothing written
    k = len(bt) // 2
    tbt[k] = w.num_pages
    for o in outs:
        o.zero_()
    hp.validate_async(desc, T, workspace=ws)
    hp.gather_batch(desc, pools, outs, workspace=ws, gated=True)
    torch.cuda.synchronize()
    assert hp.validate_verdict(desc, T, ws) == ("HP_ERR_PAGE_RANGE", k)
    for o in outs:
        assert int(torch.count_nonzero(o)) == 0


def test_gated_pipeline_two_workspaces(hp):
    """The serving loop the gate is for: step k+1's descriptor is checked on
    a second stream while step k's moves run, each step's moves wait for
    their check with an event, and two workspaces alternate. One step's
    descriptor is corrupted: only that step writes nothing."""
    w = workloads.random_small(6600, max_seqs=40, max_len=600, page_sizes=(16,), heads=(4,),
                               dims=(64,), dtypes=("f16",), alias=False)
    say("gated pipeline", w.describe())
    pool = w.make_pool(DEV)
    T = w.total_tokens
    good_bt = idx_tensor(w.block_table, DEV)
    bad = w.block_table.copy()
    bad[0] = w.num_pages + 1
    bad_bt = idx_tensor(bad, DEV)
    sp, sl = idx_tensor(w.seq_ptr, DEV), idx_tensor(w.seq_lens, DEV)
    descs = [hp.Descriptor(pool, bad_bt if k == 3 else good_bt, sp, sl) for k in range(6)]
    outs = [torch.zeros((T, w.num_heads, w.head_dim), dtype=torch.float16, device=DEV)
            for _ in descs]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    wss = [torch.empty(256, dtype=torch.uint8, device=DEV) for _ in range(2)]
    checked = [torch.cuda.Event() for _ in descs]
    moved = [torch.cuda.Event() for _ in descs]
    side.wait_stream(main)
    for k, d in enumerate(descs):
        if k >= 2:
            side.wait_event(moved[k - 2])   # workspace k % 2 is free again
        hp.validate_async(d, T, workspace=wss[k % 2], stream=side)
        checked[k].record(side)
        main.wait_event(checked[k])
        hp.gather(d, outs[k], workspace=wss[k % 2], gated=True, streaming=True, stream=main)
        moved[k].record(main)
    torch.cuda.synchronize()
    want = oracle.gather(host_bits(pool), page_size=w.page_size, num_heads=w.num_heads,
                         head_dim=w.head_dim, block_table=w.block_table, seq_ptr=w.seq_ptr,
                         seq_lens=w.seq_lens)
    for k, o in enumerate(outs):
        if k == 3:
            assert int(torch.count_nonzero(o)) == 0, "the rejected step wrote"
        else:
            assert_bits_equal(host_bits(o), want, f"step {k}")
