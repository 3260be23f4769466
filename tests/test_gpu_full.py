"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: whole-output bit comparisons where the oracle finishes in
seconds, oracle rows computed one by one (sampled) for the 1.6M-token int8
pool, plus properties that hold at any size."""
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


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    T = w.total_tokens
    starts = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    edges = np.concatenate([starts[:-1], starts[1:] - 1])
    edges = edges[(edges >= 0) & (edges < T)]
    return np.unique(np.concatenate([rng.integers(0, T, size=n), edges]))


def test_quant_dequant_and_raw_gather(hp):
    """1,024 log-normal sequences over a 200,000-page int8 pool with per-slot
    scales and a uint64 table: dequant rows sampled against the oracle
    (random rows plus every sequence's first and last row), and the raw int8
    gather of the same descriptor the same way."""
    w = workloads.quant()
    say("quant full", w.describe())
    d = OnDevice(w)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant(d.desc, out)
    torch.cuda.synchronize()
    rows = _sample_rows(w, 40000, 1)
    pool_host = host_bits(d.pool).view(np.int8)
    scales = d.scales.cpu().numpy()
    want = oracle.gather_dequant_rows(pool_host, scales, rows, **d.oracle_kw())
    got = host_bits(out[torch.from_numpy(rows).to(DEV)])
    bf16_bits_equal(got, want, "quant dequant")
    del out
    _free()
    raw = d.empty_out()
    hp.gather(d.desc, raw)
    torch.cuda.synchronize()
    want_raw = oracle.gather_rows(pool_host, rows, **d.oracle_kw())
    assert_bits_equal(host_bits(raw[torch.from_numpy(rows).to(DEV)]), want_raw.view(np.uint8),
                      "quant raw gather")
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
