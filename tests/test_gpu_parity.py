"""GPU parity: the HIP path (through the C ABI) against the CPU oracle,
element by element, on seeded inputs of oracle-friendly size. Gather and
scatter are compared bit for bit; dequant-gather with tolerance 0 (a NaN
matches any NaN); the validator's code and index exactly."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (OnDevice, assert_bits_equal, bf16_bits_equal, fill_bits, host_bits,
                      idx_tensor, oracle_gather, say)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def medium(seed, **kw):
    """Several work units per sequence and ragged tails: up to 48 sequences of
    up to 1,500 tokens, page sizes 1..64, rows of 1 B .. 8 KB."""
    args = dict(max_seqs=48, max_len=1500, page_sizes=(1, 3, 8, 16, 32, 64),
                heads=(1, 2, 8), dims=(1, 3, 16, 128))
    args.update(kw)
    return workloads.random_small(seed, **args)


# ---- gather ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(60))
def test_gather_small(hp, seed):
    w = workloads.random_small(seed)
    say("gather small", seed, w.describe())
    d = OnDevice(w)
    out = d.empty_out()
    hp.gather(d.desc, out)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), oracle_gather(d), f"seed {seed}")


@pytest.mark.parametrize("streaming", [False, True])
@pytest.mark.parametrize("seed", range(24))
def test_gather_medium(hp, seed, streaming):
    w = medium(100 + seed)
    say("gather medium", seed, streaming, w.describe())
    d = OnDevice(w)
    out = d.empty_out()
    hp.gather(d.desc, out, streaming=streaming)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), oracle_gather(d), f"seed {seed}")


def test_gather_tiny_config_and_checked(hp):
    w = workloads.tiny()
    say("gather tiny", w.describe())
    d = OnDevice(w)
    want = oracle_gather(d)
    out = d.empty_out()
    hp.gather(d.desc, out, checked=True)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), want, "tiny")
    assert out.shape == (114, 4, 8)


def test_gather_many_sequences_plan_path(hp):
    """More sequences than the per-workgroup LDS table holds: the plan pass
    writes the per-sequence offsets to the workspace first."""
    w = workloads.random_small(77, max_seqs=9000, max_len=40, page_sizes=(4, 16),
                               heads=(2,), dims=(64,), dtypes=("bf16",))
    rng = np.random.default_rng(5)
    while w.num_seqs <= 4096:
        w = workloads.random_small(int(rng.integers(1 << 30)), max_seqs=9000, max_len=40,
                                   page_sizes=(4, 16), heads=(2,), dims=(64,),
                                   dtypes=("bf16",))
    say("gather plan path", w.describe())
    d = OnDevice(w)
    out = d.empty_out()
    hp.gather(d.desc, out)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), oracle_gather(d), "plan path")


@pytest.mark.parametrize("seed", range(4))
def test_gather_plan_by_choice(hp, seed):
    """512..4096 sequences: with a workspace of hp_workspace_bytes the gather
    takes the plan pass (per-sequence offsets and a unit -> sequence map
    written once); without one, the fused scan. Both against the oracle."""
    w = workloads.random_small(80 + seed, max_seqs=4096, max_len=60, page_sizes=(4, 16),
                               heads=(1, 4), dims=(32, 128), dtypes=("bf16", "i8"),
                               num_seqs=[512, 777, 2048, 4096][seed], with_start=False)
    say("gather plan by choice", w.describe())
    d = OnDevice(w)
    want = oracle_gather(d)
    for ws in (None, torch.empty(hp.workspace_bytes(d.desc, w.total_tokens), dtype=torch.uint8,
                                 device=DEV)):
        out = d.empty_out()
        if ws is None:
            hp.gather(d.desc, out, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
        else:
            hp.gather(d.desc, out, workspace=ws)
        torch.cuda.synchronize()
        assert_bits_equal(host_bits(out), want, f"workspace {ws is not None}")


def test_plan_path_on_a_side_stream(hp):
    """The plan path's workspace, allocated by the binding, on a stream other
    than the current one: it is recorded on the call's stream, so the
    caching allocator keeps it for that stream's work. Gather and scatter
    there, then compare after the stream finished."""
    w = workloads.random_small(78, max_seqs=9000, max_len=40, page_sizes=(4, 16),
                               heads=(2,), dims=(64,), dtypes=("bf16",), num_seqs=5000,
                               alias=False)
    say("plan path, side stream", w.describe())
    d = OnDevice(w)
    out = d.empty_out()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blank = torch.zeros_like(d.pool)
    d2 = OnDevice(w, pool=blank)
    hp.gather(d.desc, out, stream=side)
    hp.scatter(d2.desc, out, stream=side)
    # work on the current stream meanwhile, allocating as it goes
    junk = [torch.ones(1 << 16, device=DEV) for _ in range(8)]
    side.synchronize()
    want = oracle_gather(d)
    assert_bits_equal(host_bits(out), want, "plan path gather, side stream")
    want_pool = oracle.scatter(host_bits(torch.zeros_like(d.pool)), want, **d.oracle_kw())
    assert_bits_equal(host_bits(blank), want_pool, "plan path scatter, side stream")
    del junk


@pytest.mark.parametrize("case", ["odd_row", "row6", "page1", "misaligned_out"])
def test_gather_vector_width_fallbacks(hp, case):
    """Rows whose byte size is not a multiple of 16, a one-token page, and an
    output view one element off 16-byte alignment."""
    geo = {"odd_row": dict(heads=(1,), dims=(3,), dtypes=("i8",)),
           "row6": dict(heads=(1,), dims=(3,), dtypes=("f16",)),
           "page1": dict(page_sizes=(1,), heads=(2,), dims=(8,), dtypes=("f32",)),
           "misaligned_out": dict(heads=(2,), dims=(8,), dtypes=("f16",))}[case]
    w = workloads.random_small(31, max_seqs=20, max_len=200, **geo)
    say("gather fallback", case, w.describe())
    d = OnDevice(w)
    if case == "misaligned_out":
        buf = torch.empty(w.total_tokens * w.num_heads * w.head_dim + 1, dtype=d.pool.dtype,
                          device=DEV)
        out = buf[1:].view(w.total_tokens, w.num_heads, w.head_dim)
    else:
        out = d.empty_out()
    hp.gather(d.desc, out)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), oracle_gather(d), case)


def test_gather_preserves_special_bit_patterns(hp):
    """NaN payloads, -0.0, subnormals and infinities are moved as bits."""
    w = workloads.random_small(41, max_seqs=12, max_len=300, dtypes=("f32",), heads=(4,),
                               dims=(16,))
    say("gather special bits", w.describe())
    pool = w.make_pool(DEV)
    specials = torch.tensor([0x7FC00001, 0xFFC12345, 0x80000000, 0x00000001, 0x807FFFFF,
                             0x7F800000, 0xFF800000, 0x7FBFFFFF], dtype=torch.int64)
    flat = pool.view(torch.int32).view(-1)
    idx = torch.arange(flat.numel(), device=DEV)
    flat.copy_(torch.where(idx % 3 == 0, specials.to(DEV)[idx % 8].to(torch.int32), flat))
    d = OnDevice(w, pool=pool)
    out = d.empty_out()
    hp.gather(d.desc, out)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), oracle_gather(d), "special bits")


def test_gather_empty_batch_and_empty_sequences(hp):
    say("gather empty batch")
    pool = torch.zeros((4, 16, 2, 8), dtype=torch.float16, device=DEV)
    z32 = torch.zeros(0, dtype=torch.int32, device=DEV)
    sp = torch.zeros(1, dtype=torch.int32, device=DEV)
    desc = hp.Descriptor(pool, z32, sp, z32)
    out = torch.empty((0, 2, 8), dtype=torch.float16, device=DEV)
    hp.gather(desc, out, checked=True)
    assert hp.validate(desc, 0) == ("HP_OK", 0)
    # three sequences, all empty, with reserved pages
    sp3 = torch.tensor([0, 1, 1, 3], dtype=torch.int32, device=DEV)
    bt = torch.tensor([2, 0, 3], dtype=torch.int32, device=DEV)
    sl = torch.zeros(3, dtype=torch.int32, device=DEV)
    d3 = hp.Descriptor(pool, bt, sp3, sl)
    hp.gather(d3, out, checked=True)
    torch.cuda.synchronize()


def test_checked_rejection_writes_nothing(hp):
    """A checked call on a descriptor that breaks an invariant returns the
    validator's code and leaves the output untouched."""
    w = workloads.tiny()
    say("checked rejection")
    d = OnDevice(w)
    bad = w.block_table.copy()
    bad[5] = w.num_pages  # one past the last page
    bad_bt = idx_tensor(bad, DEV)
    desc = hp.Descriptor(d.pool, bad_bt, d.sp, d.sl)
    out = d.empty_out()
    before = host_bits(out).copy()
    with pytest.raises(hp.HpError) as e:
        hp.gather(desc, out, checked=True)
    assert e.value.name == "HP_ERR_PAGE_RANGE"
    assert hp.validate(desc, w.total_tokens) == ("HP_ERR_PAGE_RANGE", 5)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out), before, "untouched")


# ---- scatter -----------------------------------------------------------------------------

@pytest.mark.parametrize("zero_tail", [False, True])
@pytest.mark.parametrize("seed", range(40))
def test_scatter_small(hp, seed, zero_tail):
    w = workloads.random_small(1000 + seed, alias=False, with_start=True)
    say("scatter small", seed, zero_tail, w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    want = oracle.scatter(host_bits(d.pool), host_bits(src), zero_tail=zero_tail,
                          **d.oracle_kw(with_start=True))
    hp.scatter(d.desc, src, d.ss, zero_tail=zero_tail)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, f"seed {seed}")


@pytest.mark.parametrize("zero_tail", [False, True])
@pytest.mark.parametrize("seed", range(12))
def test_scatter_medium(hp, seed, zero_tail):
    w = medium(1200 + seed, alias=False, with_start=True)
    say("scatter medium", seed, zero_tail, w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    want = oracle.scatter(host_bits(d.pool), host_bits(src), zero_tail=zero_tail,
                          **d.oracle_kw(with_start=True))
    hp.scatter(d.desc, src, d.ss, zero_tail=zero_tail, checked=True)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, f"seed {seed}")


def test_scatter_tiny_round_trip(hp):
    """The tiny config: gather to [114,4,8], scatter back into a sentinel pool;
    live slots come back, every other slot keeps the sentinel."""
    w = workloads.tiny()
    say("scatter tiny round trip")
    d = OnDevice(w)
    out = d.empty_out()
    hp.gather(d.desc, out)
    blank = fill_bits(torch.empty_like(d.pool), workloads.SENTINEL_BITS[2])
    blank_host = host_bits(blank).copy()
    d2 = OnDevice(w, pool=blank)
    hp.scatter(d2.desc, out, checked=True)
    torch.cuda.synchronize()
    want = oracle.scatter(blank_host, oracle_gather(d), **d.oracle_kw())
    assert_bits_equal(host_bits(blank), want, "round trip")


def test_scatter_plan_path(hp):
    rng = np.random.default_rng(9)
    w = None
    while w is None or w.num_seqs <= 4096:
        w = workloads.random_small(int(rng.integers(1 << 30)), max_seqs=6000, max_len=20,
                                   page_sizes=(4, 8), heads=(2,), dims=(32,),
                                   dtypes=("f16",), alias=False, with_start=True)
    say("scatter plan path", w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    want = oracle.scatter(host_bits(d.pool), host_bits(src), zero_tail=True,
                          **d.oracle_kw(with_start=True))
    hp.scatter(d.desc, src, d.ss, zero_tail=True)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, "plan path")


# ---- 1,025 .. 4,096 sequences: the fused scan with more than 4 sequences per thread ------------
#
# Up to 1,024 sequences each scan thread keeps its sequences' counts in
# registers between the scan's two passes; above that it reads them again, and
# with 64 bytes of unit per sequence the units grow to whole pages (several
# rounds of the copy loop). These sizes still take the fused (one-launch) path.

FUSED_MANY = [(1025, 16), (2500, 64), (4096, 16)]


def fused_many(seed, S, P, **kw):
    args = dict(max_len=24, page_sizes=(P,), heads=(8,), dims=(128,), dtypes=("bf16",),
                num_seqs=S)
    args.update(kw)
    return workloads.random_small(seed, **args)


@pytest.mark.parametrize("S,P", FUSED_MANY)
def test_gather_fused_many_sequences(hp, S, P):
    w = fused_many(9100 + S, S, P)
    say("gather fused many", S, P, w.describe())
    d = OnDevice(w)
    for streaming in (False, True):
        out = d.empty_out()
        hp.gather(d.desc, out, streaming=streaming)
        torch.cuda.synchronize()
        assert_bits_equal(host_bits(out), oracle_gather(d), f"S={S} P={P} streaming={streaming}")


@pytest.mark.parametrize("S,P", FUSED_MANY)
def test_scatter_fused_many_sequences(hp, S, P):
    w = fused_many(9200 + S, S, P, alias=False, with_start=True)
    say("scatter fused many", S, P, w.describe())
    d = OnDevice(w)
    src = w.make_src(DEV)
    want = oracle.scatter(host_bits(d.pool), host_bits(src), zero_tail=True,
                          **d.oracle_kw(with_start=True))
    hp.scatter(d.desc, src, d.ss, zero_tail=True)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(d.pool), want, f"S={S} P={P}")


@pytest.mark.parametrize("S,P", FUSED_MANY)
def test_dequant_fused_many_sequences(hp, S, P):
    w = fused_many(9300 + S, S, P, dtypes=("i8",))
    say("dequant fused many", S, P, w.describe())
    d = OnDevice(w)
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant(d.desc, out)
    torch.cuda.synchronize()
    want = oracle.gather_dequant(host_bits(d.pool).view(np.int8), d.scales.cpu().numpy(),
                                 **d.oracle_kw())
    bf16_bits_equal(host_bits(out), want, f"S={S} P={P}")


# ---- dequant-gather --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(30))
def test_dequant_small_and_medium(hp, seed):
    w = (workloads.random_small(3000 + seed, dtypes=("i8",)) if seed < 20
         else medium(3100 + seed, dtypes=("i8",)))
    say("dequant", seed, w.describe())
    d = OnDevice(w)
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant(d.desc, out)
    torch.cuda.synchronize()
    want = oracle.gather_dequant(host_bits(d.pool).view(np.int8), d.scales.cpu().numpy(),
                                 **d.oracle_kw())
    bf16_bits_equal(host_bits(out), want, f"seed {seed}")


def test_dequant_rounding_sweep(hp):
    """Every int8 value against scales chosen to hit round-to-nearest-even
    ties, exact values, subnormal and huge products, random bit patterns, and
    NaN/inf scales: tolerance 0 (NaN matches NaN)."""
    rng = np.random.default_rng(21)
    ties = np.array([0x3F808000, 0x3F818000, 0x3C008000, 0x3C018000, 0x00008000, 0x00018000,
                     0x7F7F8000, 0x3F800001, 0x3F807FFF, 0x3F800000], dtype=np.uint32)
    rand_bits = rng.integers(0, 1 << 32, size=6000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x80000000, 0x00000000,
                        0x00000001, 0x007FFFFF], dtype=np.uint32)
    scales = np.concatenate([ties, special, rand_bits,
                             np.geomspace(1e-3, 1e-1, 2000).astype(np.float32).view(np.uint32)])
    P, H, D = 16, 1, 256
    n_pages = -(-len(scales) // P)
    sc = np.zeros(n_pages * P, np.uint32)
    sc[: len(scales)] = scales
    pool = np.broadcast_to(np.arange(-128, 128, dtype=np.int8), (n_pages, P, H, D)).copy()
    w = workloads.Workload("sweep", "i8", P, H, D, n_pages, np.uint32,
                           np.arange(n_pages, dtype=np.uint32),
                           np.array([0, n_pages], dtype=np.uint32),
                           np.array([n_pages * P], dtype=np.uint32), values="int8")
    say("dequant rounding sweep", w.describe())
    tpool = torch.from_numpy(pool).to(DEV)
    tsc = torch.from_numpy(sc.view(np.float32)).to(DEV)
    d = OnDevice(w, pool=tpool)
    desc = hp.Descriptor(tpool, d.bt, d.sp, d.sl, scales=tsc)
    out = torch.empty((n_pages * P, H, D), dtype=torch.bfloat16, device=DEV)
    hp.gather_dequant(desc, out)
    torch.cuda.synchronize()
    want = oracle.gather_dequant(pool, sc.view(np.float32), **d.oracle_kw())
    bf16_bits_equal(host_bits(out), want, "rounding sweep")


# ---- validator ----------------------------------------------------------------------------------

def _corrupt(seed):
    rng = np.random.default_rng(seed)
    w = workloads.random_small(4000 + seed, with_start=bool(seed % 2))
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


NAMES = {"valid": "HP_OK", "seq_ptr_first": "HP_ERR_SEQPTR_FIRST",
         "seq_ptr_last": "HP_ERR_SEQPTR_LAST", "seq_ptr_order": "HP_ERR_SEQPTR_ORDER",
         "page_range": "HP_ERR_PAGE_RANGE", "seq_len": "HP_ERR_SEQ_LEN",
         "total_tokens": "HP_ERR_TOTAL_TOKENS"}


@pytest.mark.parametrize("pinned", [False, True])
@pytest.mark.parametrize("seed", range(80))
def test_validate_matches_oracle(hp, seed, pinned):
    """Pageable result: the words come through the workspace; pinned result:
    the one-workgroup check writes them into host memory itself."""
    w, bt, sp, sl, T = _corrupt(seed)
    say("validate", seed, pinned)
    dt = w.index_dtype
    pool = torch.empty((max(w.num_pages, 1), w.page_size, w.num_heads, w.head_dim),
                       dtype=torch.float16, device=DEV)
    tbt = idx_tensor(np.array(bt, dtype=dt), DEV)
    tsp = idx_tensor(np.array(sp, dtype=dt), DEV)
    tsl = idx_tensor(np.array(sl, dtype=dt), DEV)
    tss = idx_tensor(w.seq_start.astype(dt), DEV) if w.seq_start is not None else None
    desc = hp.Descriptor(pool, tbt, tsp, tsl, num_pages=w.num_pages)
    result = None
    if pinned:
        result = torch.full((2,), -1, dtype=torch.int64, pin_memory=True)  # stale words
    got = hp.validate(desc, T, tss, result=result)
    want = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages, page_size=w.page_size,
                           block_table=bt, seq_ptr=sp, seq_lens=sl, total_tokens=T,
                           seq_start=w.seq_start)
    assert got == (NAMES[want[0]], want[1]), (got, want)


def test_validate_large_block_table_first_index(hp):
    """Many violations spread over a large table: the smallest index wins."""
    say("validate first index")
    K = 1 << 20
    bt = np.arange(K, dtype=np.uint32) % 1000
    bad = np.array([K - 1, 700_001, 123_457, 999_999])
    bt[bad] = 1000
    sp = np.array([0, K], dtype=np.uint32)
    sl = np.array([K * 4], dtype=np.uint32)
    pool = torch.empty((1000, 4, 1, 16), dtype=torch.int8, device=DEV)
    desc = hp.Descriptor(pool, idx_tensor(bt, DEV), idx_tensor(sp, DEV), idx_tensor(sl, DEV))
    assert hp.validate(desc, K * 4) == ("HP_ERR_PAGE_RANGE", 123_457)
    pinned = torch.zeros(2, dtype=torch.int64, pin_memory=True)
    assert hp.validate(desc, K * 4, result=pinned) == ("HP_ERR_PAGE_RANGE", 123_457)
