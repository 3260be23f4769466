"""GPU parity of quantize-on-scatter: codes, scales and zero points bit for bit
against the oracle (the codes are integers decided by binary32 arithmetic,
and both sides take each decision with the same IEEE operations)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, host_bits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SRC = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def run_case(hp, w, src_type, asym, zero_tail, seed, scale_src=1.0, src=None):
    """Quant-scatter a seeded source (or the given one) into a pool of random
    codes and parameters; compare the whole pool, scales and zero points."""
    qw = dataclasses.replace(w, dtype="u8" if asym else "i8", values="normal", seed=seed)
    d = OnDevice(qw)
    N, P = w.num_pages, w.page_size
    g = torch.Generator(device=DEV).manual_seed(seed + 1)
    scales = torch.rand(N * P, generator=g, device=DEV) + 1.0
    zps = (torch.randint(0, 256, (N * P,), generator=g, device=DEV, dtype=torch.int32)
           .to(torch.uint8) if asym else None)
    if src is None:
        src = (torch.randn((w.total_tokens, w.num_heads, w.head_dim), generator=g, device=DEV)
               * scale_src).to(SRC[src_type])
    desc = hp.Descriptor(d.pool, d.bt, d.sp, d.sl, scales=scales)
    want_pool, want_sc, want_zp = oracle.scatter_quant(
        host_bits(d.pool).view(np.uint8 if asym else np.int8), scales.cpu().numpy(),
        host_bits(src), src_type, page_size=P, num_heads=w.num_heads, head_dim=w.head_dim,
        block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens,
        seq_start=w.seq_start, zero_points=None if zps is None else zps.cpu().numpy(),
        zero_tail=zero_tail)
    hp.scatter_quant(desc, src, d.ss, zero_points=zps, zero_tail=zero_tail)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(d.pool).view(np.uint8), want_pool.view(np.uint8)), "codes"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_sc.view(np.uint32)), \
        "scales"
    if asym:
        assert np.array_equal(zps.cpu().numpy(), want_zp), "zero points"


@pytest.mark.parametrize("zero_tail", [False, True])
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("src_type", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("seed", range(4))
def test_scatter_quant_random(hp, seed, src_type, asym, zero_tail):
    w = workloads.random_small(1700 + seed, max_seqs=20, max_len=200, page_sizes=(1, 4, 16),
                               heads=(1, 4, 8), dims=(8, 16, 128), alias=False, with_start=True)
    say("scatter quant", seed, src_type, asym, zero_tail, w.describe())
    run_case(hp, w, src_type, asym, zero_tail, 1710 + seed)


@pytest.mark.parametrize("dims", [(3,), (5,), (1,)])
def test_scatter_quant_single_value_path(hp, dims):
    """Rows whose value count is not a multiple of 8: one value per vector."""
    w = workloads.random_small(1720 + dims[0], max_seqs=16, max_len=120, page_sizes=(4, 8),
                               heads=(1, 3), dims=dims, alias=False, with_start=True)
    say("scatter quant single values", dims, w.describe())
    run_case(hp, w, "bf16", True, True, 1721)
    run_case(hp, w, "f32", False, True, 1722)


def test_scatter_quant_long_rows(hp):
    """Rows of 40 x 128 values: more vectors per thread than are held in
    registers between the two passes (the rest are read again)."""
    w = workloads.random_small(1730, max_seqs=6, max_len=40, page_sizes=(16,), heads=(40,),
                               dims=(128,), alias=False)
    say("scatter quant long rows", w.describe())
    run_case(hp, w, "f16", False, False, 1731)
    run_case(hp, w, "f32", True, True, 1732)


def test_scatter_quant_scales_spread(hp):
    """Rows of tiny and huge values (scales near the binary32 extremes)."""
    w = workloads.random_small(1740, max_seqs=10, max_len=100, page_sizes=(8,), heads=(2,),
                               dims=(64,), alias=False)
    say("scatter quant spread", w.describe())
    run_case(hp, w, "f32", False, True, 1741, scale_src=1e-30)
    run_case(hp, w, "f32", True, False, 1742, scale_src=1e30)


def test_scatter_quant_scales_spread_16bit(hp):
    """bf16 rows of tiny and huge values: scales outside [2^-100, 2^100],
    where each value is divided by the scale."""
    w = workloads.random_small(1745, max_seqs=10, max_len=100, page_sizes=(8,), heads=(2,),
                               dims=(64,), alias=False, with_start=True)
    say("scatter quant spread bf16", w.describe())
    run_case(hp, w, "bf16", False, True, 1746, scale_src=1e-30)
    run_case(hp, w, "bf16", True, False, 1747, scale_src=1e36)


# 16-bit source rows that a wave holds whole in registers (at most 4,096
# values): page sizes give units of 1, 2, 3 and 4 rows (so some waves of a
# workgroup have no row), rows run from 8 values to the largest such row.
PIPE_SHAPES = [(1, 3, 16), (2, 1, 8), (3, 2, 64), (5, 4, 128), (8, 8, 512), (16, 32, 128)]
PIPE_MODES = [("f16", False, True), ("bf16", True, True), ("f16", True, False),
              ("bf16", False, False)]


@pytest.mark.parametrize("shape", PIPE_SHAPES)
@pytest.mark.parametrize("src_type,asym,zero_tail", PIPE_MODES)
def test_scatter_quant_unit_shapes(hp, shape, src_type, asym, zero_tail):
    P, H, D = shape
    seed = 1780 + 13 * P + H + D
    w = workloads.random_small(seed, max_len=max(9, 120000 // (H * D)), page_sizes=(P,),
                               heads=(H,), dims=(D,), alias=False, with_start=True,
                               num_seqs=7 + P)
    say("scatter quant unit shapes", shape, src_type, asym, zero_tail, w.describe())
    run_case(hp, w, src_type, asym, zero_tail, seed + 1)


@pytest.mark.parametrize("asym", [False, True])
def test_scatter_quant_decode_full(hp, asym):
    """The decode batch at full size (63,540 fp16 rows of 32 x 128 values,
    12,000 pages), launched as the benchmark launches it: whole pool, scales
    and zero points against the oracle."""
    w = workloads.decode()
    say("scatter quant decode full", asym, w.describe())
    run_case(hp, w, "f16", asym, False, 1790 + asym)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("num_seqs", [200, 256, 257, 1025, 4096])
def test_scatter_quant_fused_many(hp, num_seqs):
    """Up to the fused table's 4,096 sequences: up to 256 a one-wave
    workgroup takes each slot, its lanes holding up to 4 sequences each; from
    257 four waves take a run of slots, and past 1,024 each scan thread reads
    its sequences again when it finds the workgroup's first unit."""
    w = workloads.random_small(1795 + num_seqs, max_len=24, page_sizes=(4, 16), heads=(2,),
                               dims=(64,), alias=False, with_start=True, num_seqs=num_seqs)
    say("scatter quant fused many", num_seqs, w.describe())
    run_case(hp, w, "f16", False, True, 1796)
    run_case(hp, w, "bf16", True, False, 1797)


def test_scatter_quant_plan_path(hp):
    """More sequences than the fused LDS table: the plan kernels run first."""
    rng = np.random.default_rng(1750)
    w = None
    while w is None or w.num_seqs <= 4096:
        w = workloads.random_small(int(rng.integers(1 << 30)), max_seqs=6000, max_len=6,
                                   page_sizes=(4,), heads=(2,), dims=(8,), alias=False,
                                   with_start=True)
    say("scatter quant plan path", w.describe())
    run_case(hp, w, "f16", False, True, 1751)


def test_scatter_quant_then_dequant_round_trip(hp):
    """The written codes read back through the per-block-affine dequant stay
    within a step (plus bf16 rounding) of the source."""
    w = workloads.random_small(1760, max_seqs=12, max_len=300, page_sizes=(16,), heads=(8,),
                               dims=(128,), alias=False)
    say("scatter quant round trip", w.describe())
    qw = dataclasses.replace(w, dtype="u8", values="normal")
    d = OnDevice(qw)
    N, P = w.num_pages, w.page_size
    scales = torch.zeros(N * P, device=DEV)
    zps = torch.zeros(N * P, dtype=torch.uint8, device=DEV)
    src = torch.randn((w.total_tokens, 8, 128), device=DEV).to(torch.bfloat16)
    hp.scatter_quant(hp.Descriptor(d.pool, d.bt, d.sp, d.sl, scales=scales), src,
                     zero_points=zps)
    back = torch.empty_like(src)
    hp.gather_dequant_q(hp.Descriptor(d.pool, d.bt, d.sp, d.sl), back, "per_block_affine",
                        scales, zero_points=zps)
    torch.cuda.synchronize()
    x = src.float().reshape(w.total_tokens, -1)
    step = (x.max(1).values.clamp(min=0) - x.min(1).values.clamp(max=0)) / 255
    err = (back.float().reshape(w.total_tokens, -1) - x).abs().max(1).values
    assert bool(torch.all(err <= step * 1.001 + x.abs().max(1).values * 2.0 ** -8))


def near_tie_rows(rng, count, n, asym):
    """f32 rows whose quotients x / scale sit within a few ulps of a
    half-integer or an integer: the row's extremes fix the scale (computed
    here in binary32 the way the quantizer does), the other values are
    RN((k + 1/2) * scale) or RN(k * scale) moved by -4..4 ulps."""
    rows = np.empty((count, n), np.float32)
    for r in range(count):
        mag = np.float32(np.exp2(rng.uniform(-60, 60)))
        if asym:
            lo = -mag * np.float32(rng.uniform(0.2, 1.0))
            hi = mag * np.float32(rng.uniform(0.2, 1.0))
            sc = (hi - lo) / np.float32(255)
            span = min(-lo, hi)
        else:
            amax = mag
            sc = amax / np.float32(127)
            span = amax
        kmax = int(np.floor(float(span) / float(sc))) - 1
        k = rng.integers(-kmax, kmax, n).astype(np.float64) + rng.integers(0, 2, n) * 0.5
        x = (k * float(sc)).astype(np.float32)
        m = np.maximum(np.abs(x).view(np.int32) + rng.integers(-4, 5, n).astype(np.int32), 0)
        x = np.copysign(m.view(np.float32), x)
        x = np.clip(x, -span, span)
        if asym:
            x[0], x[1] = lo, hi
        else:
            x[0] = amax if rng.integers(2) else -amax
        rows[r] = x
    return rows


@pytest.mark.parametrize("asym", [False, True])
def test_scatter_quant_near_ties(hp, asym):
    """Quotients next to the rounding boundaries, where an approximate
    division would pick the neighbouring code."""
    w = workloads.random_small(1770 + asym, max_seqs=16, max_len=120, page_sizes=(16,),
                               heads=(4,), dims=(128,), alias=False, with_start=True)
    say("scatter quant near ties", asym, w.describe())
    rng = np.random.default_rng(1771 + asym)
    rows = near_tie_rows(rng, w.total_tokens, w.num_heads * w.head_dim, asym)
    src = torch.from_numpy(rows.reshape(w.total_tokens, w.num_heads, w.head_dim)).to(DEV)
    run_case(hp, w, "f32", asym, True, 1772, src=src)
