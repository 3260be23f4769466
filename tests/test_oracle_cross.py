"""Cross-checks of the C oracle against two independent formulations on
small random descriptors (no GPU): the pure-Python slot-list brute force and
torch CPU index_select / index_copy_ over the flattened slot axis."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import brute


def _np_pool(w):
    """Host pool of workload w as integer bits (numpy), [N, P, H, D]."""
    t = w.make_pool("cpu")
    return t.view(workloads.bits_dtype(w.elem_bytes)).numpy().view(
        workloads.np_bits_dtype(w.elem_bytes))


def _np_src(w):
    t = w.make_src("cpu")
    return t.view(workloads.bits_dtype(w.elem_bytes)).numpy().view(
        workloads.np_bits_dtype(w.elem_bytes))


def _slot_ids(w, with_start=False):
    """Pool slot of every logical row, from the brute-force slot lists."""
    ids = []
    bt = [int(x) for x in w.block_table]
    sp = [int(x) for x in w.seq_ptr]
    for s in range(w.num_seqs):
        start = int(w.seq_start[s]) if (with_start and w.seq_start is not None) else 0
        slots = brute.slot_list(bt, sp, s, w.page_size)
        ids += [p * w.page_size + r for p, r in slots[start: start + int(w.seq_lens[s])]]
    return np.array(ids, dtype=np.int64)


@pytest.mark.parametrize("seed", range(60))
def test_gather_brute_and_index_select(seed):
    w = workloads.random_small(seed)
    pool = _np_pool(w)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    out = oracle.gather(pool, **kw)
    assert out.shape == (w.total_tokens, w.num_heads, w.head_dim)
    rows = brute.gather(pool.tolist(), [int(x) for x in w.block_table],
                        [int(x) for x in w.seq_ptr], [int(x) for x in w.seq_lens])
    assert out.tolist() == rows
    ids = torch.from_numpy(_slot_ids(w))
    flat = torch.from_numpy(pool.reshape(-1, w.num_heads, w.head_dim).astype(np.int64))
    ref = flat.index_select(0, ids).numpy()
    assert np.array_equal(out.astype(np.int64), ref)
    # rows gathered one by one agree with the full gather
    if w.total_tokens:
        pick = np.random.default_rng(seed).integers(0, w.total_tokens, size=7)
        assert np.array_equal(oracle.gather_rows(pool, pick, **kw), out[pick])
    # the gather reads exactly the live slots
    _, mark = oracle.gather(pool, mark_reads=True, **kw)
    assert set(np.flatnonzero(mark).tolist()) == set(_slot_ids(w).tolist())


@pytest.mark.parametrize("seed", range(60))
@pytest.mark.parametrize("zero_tail", [False, True])
def test_scatter_brute_and_index_copy(seed, zero_tail):
    # scatter destinations must be disjoint: no aliasing here
    w = workloads.random_small(1000 + seed, alias=False, with_start=True)
    pool = _np_pool(w)
    src = _np_src(w)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens,
              seq_start=w.seq_start)
    got = oracle.scatter(pool, src, zero_tail=zero_tail, **kw)
    ref4 = brute.scatter(pool.tolist(), src.tolist(), [int(x) for x in w.block_table],
                         [int(x) for x in w.seq_ptr], [int(x) for x in w.seq_lens],
                         [int(x) for x in w.seq_start], zero_tail=zero_tail)
    assert got.tolist() == ref4
    if not zero_tail:
        ids = torch.from_numpy(_slot_ids(w, with_start=True))
        flat = torch.from_numpy(pool.reshape(-1, w.num_heads, w.head_dim).astype(np.int64))
        flat.index_copy_(0, ids, torch.from_numpy(src.astype(np.int64)))
        assert np.array_equal(got.reshape(flat.shape).astype(np.int64), flat.numpy())


@pytest.mark.parametrize("seed", range(30))
def test_scatter_then_gather_round_trip(seed):
    """Scattering the gathered rows back into a sentinel pool restores every
    live slot and leaves every other slot at the sentinel."""
    w = workloads.random_small(2000 + seed, alias=False)
    pool = _np_pool(w)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    out = oracle.gather(pool, **kw)
    blank = np.full_like(pool, workloads.SENTINEL_BITS[w.elem_bytes])
    back = oracle.scatter(blank, out, **kw)
    live = _slot_ids(w)
    flat_b = back.reshape(-1, w.num_heads, w.head_dim)
    flat_p = pool.reshape(-1, w.num_heads, w.head_dim)
    assert np.array_equal(flat_b[live], flat_p[live])
    rest = np.setdiff1d(np.arange(flat_b.shape[0]), live)
    assert np.all(flat_b[rest] == workloads.SENTINEL_BITS[w.elem_bytes])


@pytest.mark.parametrize("seed", range(40))
def test_dequant_rows_and_brute(seed):
    w = workloads.random_small(3000 + seed, dtypes=("i8",))
    pool = w.make_pool("cpu").numpy()
    scales = w.make_scales("cpu").numpy()
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    got = oracle.gather_dequant(pool, scales, **kw)
    ids = _slot_ids(w)
    q = torch.from_numpy(pool.reshape(-1, w.num_heads, w.head_dim))[torch.from_numpy(ids)]
    s = torch.from_numpy(scales)[torch.from_numpy(ids)]
    ref = (q.float() * s[:, None, None]).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got.view(np.int16), ref)
    if w.total_tokens:
        pick = np.arange(w.total_tokens)[::3]
        assert np.array_equal(oracle.gather_dequant_rows(pool, scales, pick, **kw), got[pick])


@pytest.mark.parametrize("seed", range(80))
def test_validator_matches_brute_on_corrupted_descriptors(seed):
    """Random corruption of valid descriptors: the oracle reports the first
    failing check (check order, then index) of the brute-force list."""
    rng = np.random.default_rng(seed)
    w = workloads.random_small(4000 + seed, with_start=bool(seed % 2))
    bt = [int(x) for x in w.block_table]
    sp = [int(x) for x in w.seq_ptr]
    sl = [int(x) for x in w.seq_lens]
    ss = None if w.seq_start is None else [int(x) for x in w.seq_start]
    T = w.total_tokens
    for _ in range(int(rng.integers(0, 4))):
        kind = rng.integers(0, 5)
        if kind == 0 and sp:
            sp[int(rng.integers(0, len(sp)))] += int(rng.integers(-2, 3))
            sp = [max(0, x) for x in sp]
        elif kind == 1 and bt:
            bt[int(rng.integers(0, len(bt)))] = w.num_pages + int(rng.integers(0, 3))
        elif kind == 2 and sl:
            sl[int(rng.integers(0, len(sl)))] += int(rng.integers(1, 2 * w.page_size))
        elif kind == 3:
            T += int(rng.integers(-1, 2))
            T = max(0, T)
        elif kind == 4 and bt:
            bt.pop()
    got = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages,
                          page_size=w.page_size, block_table=bt, seq_ptr=sp, seq_lens=sl,
                          total_tokens=T, seq_start=ss)
    fails = brute.validate(3, 0, w.num_pages, w.page_size, bt, sp, sl, T, ss)
    assert got == (fails[0] if fails else ("valid", 0))


def test_planted_index_mistakes_fail_the_pins():
    """Plausible mistakes in the element-index formula (swapped slot/head
    strides, dropped offset, page index taken from the wrong entry, wrong
    base) each fail the worked-example pin that the oracle passes."""
    P, H, d = 3, 2, 2
    bt = [2, 0, 3, 1]
    expect = [24, 26, 28, 0, 2, 4, 36]
    good = lambda p: bt[p // P] * (H * P * d) + (p % P) * d            # noqa: E731
    mutants = [
        lambda p: bt[p // P] * (H * P * d) + (p % P) * (H * d),        # interchange strides
        lambda p: bt[p // P] * (H * P * d),                            # dropped offset
        lambda p: bt[p % len(bt)] * (H * P * d) + (p % P) * d,         # wrong table index
        lambda p: (p // P) * (H * P * d) + (p % P) * d,                # table ignored
        lambda p: bt[p // P] * (P * d) + (p % P) * d,                  # head axis dropped
    ]
    assert [good(p) for p in range(7)] == expect
    for m in mutants:
        assert [m(p) for p in range(7)] != expect


@pytest.mark.parametrize("seed", range(30))
def test_copy_pages_brute(seed):
    rng = np.random.default_rng(5000 + seed)
    w = workloads.random_small(5000 + seed, dtypes=("f16", "i8", "f64"))
    pool = _np_pool(w)
    N = w.num_pages
    n = int(rng.integers(0, max(1, N // 2) + 1))
    perm = rng.permutation(N)
    dst = perm[:n]                                   # distinct destinations
    src = rng.permutation(perm[n:])[:n] if N - n >= n else perm[n:n + n]
    src = np.resize(src, n) if n else src
    scales = rng.random(N * w.page_size).astype(np.float32)
    got, got_sc = oracle.copy_pages(pool, src, dst, page_size=w.page_size,
                                    num_heads=w.num_heads, head_dim=w.head_dim, scales=scales)
    ref, ref_sc = brute.copy_pages(pool.tolist(), scales.tolist(), [int(x) for x in src],
                                   [int(x) for x in dst])
    assert got.tolist() == ref
    assert got_sc.tolist() == ref_sc


QUANT_CASES = [("per_tensor", 0), ("per_channel", 1), ("per_channel", 2),
               ("per_block_affine", 0)]


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("scheme,axis", QUANT_CASES)
@pytest.mark.parametrize("signed", [True, False])
@pytest.mark.parametrize("with_zp", [False, True])
def test_dequant_schemes_match_library_arithmetic(seed, scheme, axis, signed, with_zp):
    """bf16(fp32(q - zp) * scale) under each scheme equals torch CPU's
    ((q - zp).float() * scale).to(bfloat16), with the scheme's parameter
    broadcast over the logical tensor."""
    w = workloads.random_small(6000 + seed, dtypes=("i8",))
    rng = np.random.default_rng(seed)
    N, P, H, D = w.num_pages, w.page_size, w.num_heads, w.head_dim
    qdt = np.int8 if signed else np.uint8
    lo, hi = (-128, 128) if signed else (0, 256)
    pool = rng.integers(lo, hi, size=(N, P, H, D)).astype(qdt)
    n = {"per_tensor": 1, "per_channel": H if axis == 1 else D, "per_block_affine": N * P}[scheme]
    scales = rng.uniform(1e-3, 1e-1, n).astype(np.float32)
    zp = rng.integers(lo, hi, n).astype(qdt) if with_zp else None
    kw = dict(page_size=P, num_heads=H, head_dim=D, block_table=w.block_table,
              seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    got = oracle.gather_dequant_scheme(pool, scheme, axis, scales, zp, **kw)
    ids = torch.from_numpy(_slot_ids(w))
    q = torch.from_numpy(pool.reshape(-1, H, D).astype(np.int32))[ids]
    s = torch.from_numpy(scales)
    z = torch.from_numpy(zp.astype(np.int32)) if with_zp else torch.zeros(n, dtype=torch.int32)
    if scheme == "per_tensor":
        sb, zb = s.view(1, 1, 1), z.view(1, 1, 1)
    elif scheme == "per_channel" and axis == 1:
        sb, zb = s.view(1, H, 1), z.view(1, H, 1)
    elif scheme == "per_channel":
        sb, zb = s.view(1, 1, D), z.view(1, 1, D)
    else:
        sb, zb = s[ids].view(-1, 1, 1), z[ids].view(-1, 1, 1)
    ref = ((q - zb).float() * sb).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got.view(np.int16), ref)


def test_dequant_scheme_per_block_affine_is_the_per_slot_path():
    """Per-block-affine on axis 0 with block_size == page_size coincides with
    the per-page-slot parameters ([Hurray] Per-scheme composition)."""
    w = workloads.random_small(6100, dtypes=("i8",))
    pool = w.make_pool("cpu").numpy()
    scales = w.make_scales("cpu").numpy()
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    assert np.array_equal(oracle.gather_dequant_scheme(pool, "per_block_affine", 0, scales, **kw),
                          oracle.gather_dequant(pool, scales, **kw))
