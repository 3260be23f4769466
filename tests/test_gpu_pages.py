"""GPU parity of the copy-on-write page copy against the oracle, and the
copy-on-write scenario run end to end through the GPU path."""
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


def _copies(w, seed):
    """Distinct destinations that are never sources."""
    rng = np.random.default_rng(seed)
    N = w.num_pages
    perm = rng.permutation(N)
    n = int(rng.integers(1, max(2, N // 3)))
    dst = perm[:n]
    src = rng.choice(perm[n:], size=n, replace=True) if N > n else perm[:0]
    return src.astype(w.index_dtype), dst[: len(src)].astype(w.index_dtype)


@pytest.mark.parametrize("seed", range(16))
def test_copy_pages(hp, seed):
    w = workloads.random_small(900 + seed, max_seqs=10, max_len=200,
                               dtypes=("f16", "i8", "f32", "bf16"))
    say("copy pages", seed, w.describe())
    d = OnDevice(w)
    src, dst = _copies(w, seed)
    before = host_bits(d.pool)
    sc_before = d.scales.cpu().numpy() if d.scales is not None else None
    want, want_sc = oracle.copy_pages(before, src, dst, page_size=w.page_size,
                                      num_heads=w.num_heads, head_dim=w.head_dim,
                                      scales=sc_before)
    hp.copy_pages(d.desc, idx_tensor(src, DEV), idx_tensor(dst, DEV), checked=bool(seed % 2))
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, "pool")
    if sc_before is not None:
        assert_bits_equal(d.scales.cpu().numpy().view(np.uint32), want_sc.view(np.uint32),
                          "scales")


@pytest.mark.parametrize("count", [3, 35])
def test_copy_pages_batch(hp, count):
    w = workloads.random_small(950 + count, max_seqs=8, max_len=120, dtypes=("i8",))
    say("copy pages batch", count, w.describe())
    d = OnDevice(w)
    ms = [dataclasses.replace(w, seed=w.seed * 100 + i) for i in range(count)]
    pools = [m.make_pool(DEV) for m in ms]
    scales = [m.make_scales(DEV) for m in ms]
    src, dst = _copies(w, count)
    want = [oracle.copy_pages(host_bits(p), src, dst, page_size=w.page_size,
                              num_heads=w.num_heads, head_dim=w.head_dim,
                              scales=s.cpu().numpy()) for p, s in zip(pools, scales)]
    hp.copy_pages_batch(d.desc, pools, scales, idx_tensor(src, DEV), idx_tensor(dst, DEV))
    torch.cuda.synchronize()
    for i, (p, s, (wp, ws)) in enumerate(zip(pools, scales, want)):
        assert_bits_equal(host_bits(p), wp, f"pool {i}")
        assert_bits_equal(s.cpu().numpy().view(np.uint32), ws.view(np.uint32), f"scales {i}")


def test_copy_pages_checked_rejects_out_of_range(hp):
    w = workloads.tiny()
    say("copy pages checked")
    d = OnDevice(w)
    before = host_bits(d.pool).copy()
    src = np.array([3, 5, 20], dtype=np.uint32)     # 20 == num_pages
    dst = np.array([1, 2, 4], dtype=np.uint32)
    with pytest.raises(hp.HpError) as e:
        hp.copy_pages(d.desc, idx_tensor(src, DEV), idx_tensor(dst, DEV), checked=True)
    assert e.value.name == "HP_ERR_PAGE_RANGE"
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), before, "untouched")


def test_copy_on_write_scenario(hp):
    """[Day51] copy-on-write on the GPU: two requests share a 24-token prompt
    (pages 0, 1; page 1 half full); request E's page 1 is copied to page 4,
    E's table is repointed and E appends a token at position 24. The GPU's
    gather of both requests equals the oracle's result of the same steps."""
    P, H, D, N = 16, 8, 128, 8
    w = workloads.Workload("cow", "bf16", P, H, D, N, np.uint32,
                           np.array([0, 1, 2, 0, 1, 3], np.uint32),
                           np.array([0, 3, 6], np.uint32), np.array([24, 24], np.uint32))
    say("copy on write scenario")
    d = OnDevice(w)
    pool0 = host_bits(d.pool).copy()
    kw = dict(page_size=P, num_heads=H, head_dim=D)
    hp.copy_pages(d.desc, idx_tensor(np.array([1], np.uint32), DEV),
                  idx_tensor(np.array([4], np.uint32), DEV))
    bt_e = np.array([0, 4, 3], np.uint32)
    new_row = torch.randn((1, H, D), device=DEV).to(torch.bfloat16)
    de = hp.Descriptor(d.pool, idx_tensor(bt_e, DEV), idx_tensor(np.array([0, 3], np.uint32), DEV),
                       idx_tensor(np.array([1], np.uint32), DEV))
    hp.scatter(de, new_row, idx_tensor(np.array([24], np.uint32), DEV), zero_tail=True)
    bt_all = np.array([0, 1, 2, 0, 4, 3], np.uint32)
    lens = np.array([24, 25], np.uint32)
    dall = hp.Descriptor(d.pool, idx_tensor(bt_all, DEV), d.sp, idx_tensor(lens, DEV))
    out = torch.empty((49, H, D), dtype=torch.bfloat16, device=DEV)
    hp.gather(dall, out, checked=True)
    torch.cuda.synchronize()
    p1, _ = oracle.copy_pages(pool0, [1], [4], **kw)
    p2 = oracle.scatter(p1, host_bits(new_row), block_table=bt_e, seq_ptr=[0, 3], seq_lens=[1],
                        seq_start=[24], zero_tail=True, **kw)
    want = oracle.gather(p2, block_table=bt_all, seq_ptr=w.seq_ptr, seq_lens=lens, **kw)
    got = host_bits(out)
    assert_bits_equal(got, want, "scenario")
    assert np.array_equal(got[:24], got[24:48])      # E's prefix == D's
    assert_bits_equal(host_bits(d.pool)[1], pool0[1], "shared page untouched")


def test_copy_pages_decode_pool(hp):
    """The decode pool at full size (12,000 pages of 16 x 32 x 128 fp16 =
    128 KiB) in the benchmark's launch: 1,024 referenced pages copied to
    pages no sequence references. The whole pool afterwards equals the
    oracle's, bit for bit."""
    w = workloads.decode()
    say("copy pages decode pool", w.describe())
    d = OnDevice(w)
    free = np.setdiff1d(np.arange(w.num_pages), w.block_table.astype(np.int64))
    rng = np.random.default_rng(6)
    src = rng.choice(w.block_table.astype(np.int64), 1024, replace=False).astype(np.uint32)
    dst = rng.choice(free, 1024, replace=False).astype(np.uint32)
    before = host_bits(d.pool)
    want, _ = oracle.copy_pages(before, src, dst, page_size=w.page_size,
                                num_heads=w.num_heads, head_dim=w.head_dim)
    del before
    hp.copy_pages(d.desc, idx_tensor(src, DEV), idx_tensor(dst, DEV))
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, "pool")
