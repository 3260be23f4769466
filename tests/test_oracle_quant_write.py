"""Pins of the quantize-on-scatter oracle (CPU only).

The pages say where a written slot's parameters live ([Hurray] Per-page-slot
parameters) but not how they are computed; the oracle's reading is absmax
int8 (symmetric) and min/max uint8 with a zero point (asymmetric), each step a
binary32 operation rounded to nearest even. Pinned here by what holds for any
correct quantizer of that kind: codes in range with the extreme value at the
end of the range, reconstruction within half a step, nearest-even rounding
of the binary32 quotient, invariance under power-of-two scaling,
monotonicity, the placement of rows and parameters (against the brute-force
slot list), and a round trip through the pinned scheme dequant.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import brute


def rows(seed, count=200, n=96):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(n)
        elif kind == 1:
            x = rng.uniform(0.5, 3.0, n)                    # all positive
        elif kind == 2:
            x = -rng.exponential(2.0, n)                    # all negative
        else:
            x = rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6)
        out.append(x.astype(np.float32))
    return out


def test_zero_row_and_single_value():
    q, s, _ = oracle.quantize_row(np.zeros(8, np.float32))
    assert s == 0 and np.all(q == 0)
    q, s, z = oracle.quantize_row(np.zeros(8, np.float32), asym=True)
    assert s == 0 and z == 0 and np.all(q == 0)
    x = np.zeros(8, np.float32)
    x[3] = -0.75
    q, s, _ = oracle.quantize_row(x)
    assert q[3] == -127 and np.all(np.delete(q, 3) == 0) and s == np.float32(0.75) / np.float32(127)


@pytest.mark.parametrize("asym", [False, True])
def test_codes_in_range_and_extremes(asym):
    for x in rows(1):
        q, s, z = oracle.quantize_row(x, asym)
        q = q.astype(np.int64)
        if not asym:
            assert q.min() >= -127 and q.max() <= 127
            assert np.abs(q).max() == 127                   # the largest |x| maps to +-127
            assert q[np.argmax(np.abs(x))] == np.sign(x[np.argmax(np.abs(x))]) * 127
        else:
            assert q.min() >= 0 and q.max() <= 255
            if x.min() < 0:
                assert q[np.argmin(x)] == 0                 # the lowest value maps to code 0
            if x.max() > 0:
                assert q[np.argmax(x)] in (254, 255)        # the highest to the top step
            assert 0 <= z <= 255


@pytest.mark.parametrize("asym", [False, True])
def test_reconstruction_within_half_a_step(asym):
    for x in rows(2):
        q, s, z = oracle.quantize_row(x, asym)
        x64, s64 = x.astype(np.float64), float(s)
        rec = (q.astype(np.float64) - (z or 0)) * s64
        # symmetric: half a step (plus the quotient's rounding); asymmetric:
        # the zero point's own rounding adds up to another half step
        bound = s64 * (0.5 if not asym else 1.0) * (1 + 2.0 ** -20) + 1e-300
        assert np.all(np.abs(x64 - rec) <= bound)


@pytest.mark.parametrize("asym", [False, True])
def test_codes_are_nearest_even_of_the_binary32_quotient(asym):
    """Each code is the binary32 quotient x / scale rounded to the nearest
    integer, ties to even (numpy's float32 division and rint as the library
    steps), then shifted by the zero point and clamped."""
    for x in rows(3):
        q, s, z = oracle.quantize_row(x, asym)
        quot = np.rint(x / np.float32(s)).astype(np.int64)
        if not asym:
            assert np.array_equal(q.astype(np.int64), np.clip(quot, -127, 127))
        else:
            assert np.array_equal(q.astype(np.int64), np.clip(quot + z, 0, 255))


def test_ties_round_to_even():
    """Quotients of exactly k + 0.5 go to the even neighbour."""
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 63.5], np.float32)  # amax 127: scale 1
    q, s, _ = oracle.quantize_row(x)
    assert s == 1.0
    assert q.tolist() == [127, 0, 2, 2, 0, -2, 64]


@pytest.mark.parametrize("asym", [False, True])
def test_power_of_two_scaling(asym):
    for x in rows(4, count=60):
        for k in (-8, -1, 3, 10):
            q1, s1, z1 = oracle.quantize_row(x, asym)
            q2, s2, z2 = oracle.quantize_row(x * np.float32(2.0 ** k), asym)
            if s1 == 0 or not np.isfinite(s2) or abs(float(s1)) < 1e-30:
                continue
            assert np.array_equal(q1, q2) and z1 == z2 and s2 == s1 * np.float32(2.0 ** k)


@pytest.mark.parametrize("asym", [False, True])
def test_monotone(asym):
    for x in rows(5, count=60):
        q, _, _ = oracle.quantize_row(x, asym)
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(q.astype(np.int64)[order]) >= 0)


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("zero_tail", [False, True])
@pytest.mark.parametrize("seed", range(15))
def test_scatter_quant_places_rows_and_parameters(seed, zero_tail, asym):
    """Each new row is quantized on its own and lands in the slot the
    brute-force slot list names; its scale (and zero point) at that slot;
    with zero_tail the rest of the last written page is cleared; every other
    slot is unchanged."""
    w = workloads.random_small(7000 + seed, alias=False, with_start=True, dtypes=("f16",),
                               heads=(1, 2, 3), dims=(1, 2, 4, 8))
    rng = np.random.default_rng(seed)
    N, P, H, D = w.num_pages, w.page_size, w.num_heads, w.head_dim
    qdt = np.uint8 if asym else np.int8
    pool = rng.integers(0, 256, size=(N, P, H, D)).astype(np.uint8).view(qdt)
    scales = rng.uniform(1, 2, N * P).astype(np.float32)
    zps = rng.integers(0, 256, N * P).astype(np.uint8) if asym else None
    src = (rng.standard_normal((w.total_tokens, H, D)) * 3).astype(np.float16)
    got_pool, got_sc, got_zp = oracle.scatter_quant(
        pool, scales, src.view(np.uint16), "f16", page_size=P, num_heads=H, head_dim=D,
        block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens,
        seq_start=w.seq_start, zero_points=zps, zero_tail=zero_tail)
    want_pool, want_sc = pool.copy(), scales.copy()
    want_zp = None if zps is None else zps.copy()
    row = 0
    for s in range(w.num_seqs):
        slots = brute.slot_list(w.block_table.tolist(), w.seq_ptr.tolist(), s, P)
        start = int(w.seq_start[s])
        L = int(w.seq_lens[s])
        for i in range(L):
            page, slot = slots[start + i]
            q, sc, z = oracle.quantize_row(src[row].astype(np.float32).ravel(), asym)
            want_pool[page, slot] = q.reshape(H, D)
            want_sc[page * P + slot] = sc
            if asym:
                want_zp[page * P + slot] = z
            row += 1
        if zero_tail and L:
            end = start + L
            page = slots[end - 1][0]
            for slot in range((end - 1) % P + 1, P):
                want_pool[page, slot] = 0
                want_sc[page * P + slot] = 0
                if asym:
                    want_zp[page * P + slot] = 0
    assert np.array_equal(got_pool.view(np.uint8), want_pool.view(np.uint8))
    assert np.array_equal(got_sc.view(np.uint32), want_sc.view(np.uint32))
    if asym:
        assert np.array_equal(got_zp, want_zp)


@pytest.mark.parametrize("asym", [False, True])
def test_round_trip_through_scheme_dequant(asym):
    """Quantize-on-scatter then the per-block-affine dequant (scales and zero
    points per slot) reproduces every written value within a step."""
    w = workloads.random_small(7100, alias=False, dtypes=("bf16",), heads=(2,), dims=(16,),
                               max_seqs=8, max_len=80)
    rng = np.random.default_rng(7101)
    N, P, H, D = w.num_pages, w.page_size, w.num_heads, w.head_dim
    qdt = np.uint8 if asym else np.int8
    pool = np.zeros((N, P, H, D), qdt)
    src = rng.standard_normal((w.total_tokens, H, D)).astype(np.float32)
    qpool, sc, zp = oracle.scatter_quant(
        pool, np.zeros(N * P, np.float32), src.view(np.uint32), "f32", page_size=P,
        num_heads=H, head_dim=D, block_table=w.block_table, seq_ptr=w.seq_ptr,
        seq_lens=w.seq_lens, zero_points=np.zeros(N * P, np.uint8) if asym else None)
    deq = oracle.gather_dequant_scheme(qpool, "per_block_affine", 0, sc, zp, page_size=P,
                                       num_heads=H, head_dim=D, block_table=w.block_table,
                                       seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
    back = oracle.decode(deq, "bf16")
    row_scale = np.array([np.abs(r).max() / 127 if not asym else np.ptp(np.append(r, 0)) / 255
                          for r in src.reshape(len(src), -1)]) if len(src) else np.zeros(0)
    err = np.abs(back.reshape(len(src), -1) - src.reshape(len(src), -1)).max(axis=1) \
        if len(src) else np.zeros(0)
    # a step (asymmetric) or half a step, plus bf16's own rounding of the value
    tol = row_scale * (1.0 if asym else 0.5) * 1.001 + 2.0 ** -8 * np.abs(src).reshape(
        len(src), -1).max(axis=1) if len(src) else np.zeros(0)
    assert np.all(err <= tol)
