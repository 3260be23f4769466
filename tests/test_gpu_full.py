"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: whole-output bit comparisons (the 1.6M-token int8 pool in
ranges of sequences, each against the oracle on its own slice of the
table), plus properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (OnDevice, assert_bits_equal, bf16_bits_equal, host_bits, oracle_gather,
                      say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_gather_and_round_trip(hp):
    """64 sequences of 1..2048 tokens, 32 heads x 128 fp16, 12,000 pages."""
    w = workloads.decode()
    say("decode full", w.describe())
    d = OnDevice(w)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    out = d.empty_out()
    hp.gather(d.desc, out, streaming=True)  # unique pages: the benchmark's launch
    torch.cuda.synchronize()
    pool_host = host_bits(d.pool)
    want = oracle.gather(pool_host, **d.oracle_kw())
    assert_bits_equal(host_bits(out), want, "decode gather")
    # scatter the logical tensor back into a zeroed pool: the oracle's
    # scatter of the same rows into the same zero pool, bit for bit
    zero = torch.zeros_like(d.pool)
    d2 = OnDevice(w, pool=zero)
    hp.scatter(d2.desc, out)
    torch.cuda.synchronize()
    want_pool = oracle.scatter(np.zeros_like(pool_host), want, **d.oracle_kw())
    assert_bits_equal(host_bits(zero), want_pool, "decode scatter")
    del d, d2, out, zero
    _free()


def test_prefix_gather(hp):
    """256 sequences sharing 64 aliased prefix pages: whole output against the
    oracle, and the 1,024 prefix rows of every sequence bit-identical."""
    w = workloads.prefix()
    say("prefix full", w.describe())
    d = OnDevice(w)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    out = d.empty_out()
    hp.gather(d.desc, out)
    torch.cuda.synchronize()
    got = host_bits(out)
    assert_bits_equal(got, oracle_gather(d), "prefix gather")
    starts = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])[:-1]
    first = got[:1024]
    for s0 in starts:
        assert np.array_equal(got[s0: s0 + 1024], first)
    del d, out
    _free()


def test_append_scatter_zero_tail(hp):
    """512 one-token appends into partial trailing pages plus an 8,192-token
    prefill into fresh pages, tails zeroed: the whole 1.97 GB pool against
    the oracle's scatter."""
    w = workloads.append()
    say("append full", w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    assert hp.validate(d.desc, w.total_tokens, d.ss) == ("HP_OK", 0)
    before = host_bits(d.pool)
    want = oracle.scatter(before, host_bits(src), zero_tail=True, **d.oracle_kw(with_start=True))
    del before
    hp.scatter(d.desc, src, d.ss, zero_tail=True)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, "append scatter")
    del d, src, want
    _free()


def _seq_chunks(w, per):
    """(first sequence, end sequence, first row, end row) of consecutive
    sequence ranges of `per` sequences each, covering the whole batch."""
    tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    for s0 in range(0, w.num_seqs, per):
        s1 = min(s0 + per, w.num_seqs)
        yield s0, s1, int(tok[s0]), int(tok[s1])


def _sub_kw(w, s0, s1):
    """Oracle arguments for sequences [s0, s1) on their own: their slice of
    the block table, seq_ptr rebased to 0 and their counts."""
    sp = w.seq_ptr.astype(np.int64)
    return dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                block_table=w.block_table[sp[s0]: sp[s1]],
                seq_ptr=(sp[s0: s1 + 1] - sp[s0]).astype(np.uint64),
                seq_lens=w.seq_lens[s0:s1])


def test_quant_dequant_and_raw_gather(hp):
    """1,024 log-normal sequences over a 200,000-page int8 pool with per-slot
    scales and a uint64 table: every one of the 1.65M dequantised rows, and
    every row of the raw int8 gather of the same descriptor, against the
    oracle. The oracle runs on ranges of 64 sequences (each with its own
    slice of the table), compared with the matching rows of the one GPU
    launch over the whole batch."""
    w = workloads.quant()
    say("quant full", w.describe())
    d = OnDevice(w)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    pool_host = host_bits(d.pool).view(np.int8)
    scales = d.scales.cpu().numpy()
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant(d.desc, out)
    torch.cuda.synchronize()
    rows = 0
    for s0, s1, r0, r1 in _seq_chunks(w, 64):
        want = oracle.gather_dequant(pool_host, scales, **_sub_kw(w, s0, s1))
        bf16_bits_equal(host_bits(out[r0:r1]), want, f"quant dequant, sequences {s0}..{s1 - 1}")
        rows += r1 - r0
    assert rows == w.total_tokens
    del out
    _free()
    raw = d.empty_out()
    hp.gather(d.desc, raw)
    torch.cuda.synchronize()
    for s0, s1, r0, r1 in _seq_chunks(w, 64):
        want_raw = oracle.gather(pool_host, **_sub_kw(w, s0, s1))
        assert_bits_equal(host_bits(raw[r0:r1]), want_raw.view(np.uint8),
                          f"quant raw gather, sequences {s0}..{s1 - 1}")
    say("quant full: all", w.total_tokens, "rows bit-exact (dequant and raw gather)")
    del d, raw
    _free()


def test_pool_beyond_4gib_uses_64bit_offsets(hp):
    """An int8 pool of 300,000 pages x 16 x 8 x 128 (4.9 GB) with a uint64
    table whose pages lie mostly past the 4 GiB byte offset: gather and
    dequant against the oracle on the whole output."""
    rng = np.random.default_rng(44)
    N, P, H, D = 300_000, 16, 8, 128
    lens = rng.integers(1, 600, size=40)
    counts = (lens + P - 1) // P
    high = rng.permutation(np.arange(270_000, N))[: int(counts.sum())]
    high[::7] = rng.integers(0, 1000, size=len(high[::7]))  # a few low pages too
    w = workloads.Workload("pool5g", "i8", P, H, D, N, np.uint64, high.astype(np.uint64),
                           np.concatenate([[0], np.cumsum(counts)]).astype(np.uint64),
                           lens.astype(np.uint64), values="int8", with_scales=True, seed=44)
    say("pool > 4 GiB", w.describe())
    d = OnDevice(w)
    out = d.empty_out()
    hp.gather(d.desc, out, streaming=True)  # unique pages: the benchmark's launch
    torch.cuda.synchronize()
    pool_host = host_bits(d.pool).view(np.int8)
    assert_bits_equal(host_bits(out).view(np.int8),
                      oracle.gather(pool_host, **d.oracle_kw()), "gather > 4 GiB")
    outq = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant(d.desc, outq)
    torch.cuda.synchronize()
    bf16_bits_equal(host_bits(outq),
                    oracle.gather_dequant(pool_host, d.scales.cpu().numpy(), **d.oracle_kw()),
                    "dequant > 4 GiB")
    del d, out, outq
    _free()


@pytest.mark.parametrize("zero_tail", [False, True])
def test_large_ragged_scatter_streams(hp, zero_tail):
    """A scatter moving more than the Infinity Cache holds (streamed source,
    8 KB units) with ragged lengths, start offsets and tail zeroing: the
    whole pool against the oracle."""
    w = workloads.random_small(515 + int(zero_tail), max_seqs=96, max_len=2000,
                               page_sizes=(16,), heads=(32,), dims=(128,), dtypes=("f16",),
                               alias=False, with_start=True)
    if 2 * w.total_tokens * w.row_bytes < (256 << 20):
        pytest.skip("draw too small for the streaming path")
    say("large scatter", zero_tail, w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    want = oracle.scatter(host_bits(d.pool), host_bits(src), zero_tail=zero_tail,
                          **d.oracle_kw(with_start=True))
    hp.scatter(d.desc, src, d.ss, zero_tail=zero_tail)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, "large scatter")
    del d, src, want
    _free()


def test_scatter_into_a_page_beyond_4gib(hp):
    """One page of 524,288 slots x 16 KiB rows (8 GiB, f16 64 heads x 128): a
    scatter of 16 rows starting at slot 300,000, whose byte offset inside the
    page (4.9e9) does not fit 32 bits, with the page's tail zeroed. The rows
    land at their slot, the tail is zero, and every other byte keeps the
    sentinel (in particular the slots a 32-bit offset would wrap to)."""
    P, H, D, start, n = 524_288, 64, 128, 300_000, 16
    row = H * D  # f16 elements
    pool = torch.empty((1, P, H, D), dtype=torch.float16, device=DEV)
    sentinel = workloads.SENTINEL_BITS[2]
    fill = workloads._signed(sentinel, 2)
    pool.view(torch.int16).fill_(fill)
    say("scatter, page beyond 4 GiB", P * row * 2, "bytes per page")
    w = workloads.Workload("bigpage", "f16", P, H, D, 1, np.uint64, np.zeros(1, np.uint64),
                           np.array([0, 1], np.uint64), np.array([n], np.uint64),
                           seq_start=np.array([start], np.uint64), seed=45)
    d = OnDevice(w, pool=pool)
    src = w.make_src(DEV)
    hp.scatter(d.desc, src, d.ss, zero_tail=True)
    torch.cuda.synchronize()
    flat = pool.view(torch.int16).view(P, row)
    assert torch.equal(flat[start: start + n], src.view(torch.int16).view(n, row))
    assert bool((flat[start + n:] == 0).all())
    assert bool((flat[:start] == fill).all())
    wrapped = (start * row * 2) % (1 << 32) // (row * 2)
    assert wrapped < start and bool((flat[wrapped: wrapped + n] == fill).all())
    del pool, flat, d, src
    _free()
