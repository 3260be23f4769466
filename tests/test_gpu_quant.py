"""GPU parity of the dequant-gather under every quantization scheme a
block-paged reader accepts ([Hurray] Quantization Compatibility, Per-scheme
composition): per-tensor, per-channel along the head or head_dim axis, and
per-block-affine with one block per page, each with and without zero points,
over int8 and uint8 pools. Bit-exact against the oracle (tolerance 0; any NaN
matches any NaN)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, bf16_bits_equal, host_bits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [("per_tensor", 0), ("per_channel", 1), ("per_channel", 2), ("per_block_affine", 0)]


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def n_params(scheme, axis, w):
    if scheme == "per_tensor":
        return 1
    if scheme == "per_channel":
        return w.num_heads if axis == 1 else w.head_dim
    return w.num_pages * w.page_size


def make_params(w, scheme, axis, seed, with_zp, extreme=False):
    """Seeded fp32 scales (uniform in [1e-3, 1e-1), or a mix of special values
    when `extreme`) and zero points over the pool's whole integer range."""
    rng = np.random.default_rng(seed)
    n = n_params(scheme, axis, w)
    sc = rng.uniform(1e-3, 1e-1, size=n).astype(np.float32)
    if extreme:
        special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -3e-39, 1.5e-45,
                            3.0e38, -2.5e38, 1.0, -7.0], dtype=np.float32)
        pick = rng.random(n) < 0.6
        sc[pick] = rng.choice(special, size=int(pick.sum()))
    zp = None
    if with_zp:
        lo, hi = (0, 256) if w.dtype == "u8" else (-128, 128)
        zp = rng.integers(lo, hi, size=n).astype(np.uint8 if w.dtype == "u8" else np.int8)
        if n > 2:
            zp[:2] = (lo, hi - 1)   # both ends of the range
    return sc, zp


def run_case(hp, w, scheme, axis, seed, with_zp, extreme=False):
    d = OnDevice(w)
    sc, zp = make_params(w, scheme, axis, seed, with_zp, extreme)
    sc_dev = torch.from_numpy(sc).to(DEV)
    zp_dev = None if zp is None else torch.from_numpy(zp).to(DEV)
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant_q(d.desc, out, scheme, sc_dev, axis=axis, zero_points=zp_dev)
    torch.cuda.synchronize()
    pool = host_bits(d.pool).view(np.uint8 if w.dtype == "u8" else np.int8)
    want = oracle.gather_dequant_scheme(pool, scheme, axis, sc, zp, **d.oracle_kw())
    bf16_bits_equal(host_bits(out), want, f"{scheme} axis {axis} zp={with_zp}")


@pytest.mark.parametrize("with_zp", [False, True])
@pytest.mark.parametrize("scheme,axis", CASES)
@pytest.mark.parametrize("seed", range(6))
def test_scheme_random(hp, seed, scheme, axis, with_zp):
    w = workloads.random_small(900 + seed, max_seqs=24, max_len=300, page_sizes=(1, 3, 8, 16),
                               heads=(1, 3, 8), dims=(1, 2, 5, 16, 128), dtypes=("i8", "u8"))
    say("dequant scheme", seed, scheme, axis, with_zp, w.describe())
    run_case(hp, w, scheme, axis, seed, with_zp)


@pytest.mark.parametrize("scheme,axis", CASES)
def test_scheme_special_scales(hp, scheme, axis):
    """Zero, signed zero, infinities, NaN, subnormal and near-overflow scales:
    the products round (or overflow) exactly as the oracle's."""
    w = workloads.random_small(950, max_seqs=16, max_len=200, page_sizes=(16,), heads=(8,),
                               dims=(64,), dtypes=("i8",))
    say("dequant scheme special", scheme, axis, w.describe())
    run_case(hp, w, scheme, axis, 951, with_zp=True, extreme=True)


def test_scheme_plan_path(hp):
    """More sequences than the LDS table holds: the plan kernels feed the
    general dequant kernel."""
    rng = np.random.default_rng(21)
    w = None
    while w is None or w.num_seqs <= 4096:
        w = workloads.random_small(int(rng.integers(1 << 30)), max_seqs=7000, max_len=12,
                                   page_sizes=(4,), heads=(2,), dims=(16,), dtypes=("u8",))
    say("dequant scheme plan path", w.describe())
    run_case(hp, w, "per_channel", 2, 22, with_zp=True)


@pytest.mark.parametrize("scheme,axis,heads,dim,dtype", [
    ("per_channel", 1, 2100, 2, "u8"),     # more heads than the LDS table holds
    ("per_channel", 2, 1, 2304, "i8"),     # head_dim beyond the LDS table
    ("per_channel", 2, 2, 2051, "u8"),     # odd head_dim: per-element parameters
    ("per_channel", 1, 2049, 3, "i8"),
])
def test_scheme_tables_in_global_memory(hp, scheme, axis, heads, dim, dtype):
    """Per-channel tables with more than 2,048 entries are read from global
    memory instead of LDS."""
    w = workloads.random_small(980 + heads + dim, max_seqs=6, max_len=20, page_sizes=(4,),
                               heads=(heads,), dims=(dim,), dtypes=(dtype,))
    say("dequant scheme global table", scheme, axis, w.describe())
    run_case(hp, w, scheme, axis, 981, with_zp=True)


@pytest.mark.parametrize("axis", [1, 2])
def test_scheme_lds_at_limit(hp, axis):
    """4,096 sequences (the most the in-LDS sequence table takes) with a
    2,048-entry channel table: 48 KiB + 16 KiB of LDS in one workgroup."""
    rng = np.random.default_rng(990 + axis)
    S, P = 4096, 4
    H, D = (2048, 1) if axis == 1 else (1, 2048)
    lens = rng.integers(0, 4, size=S)
    counts = (lens + P - 1) // P
    K = int(counts.sum())
    bt = rng.permutation(K + 3)[:K].astype(np.uint32)
    sp = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    w = workloads.Workload("lds_limit", "u8", P, H, D, K + 3, np.uint32, bt, sp,
                           lens.astype(np.uint32), values="normal", seed=992)
    say("dequant scheme lds limit", axis, w.describe())
    run_case(hp, w, "per_channel", axis, 993, with_zp=True)


def test_per_block_affine_symmetric_matches_per_slot(hp):
    """Per-block-affine int8 with all-zero zero points is the per-slot scheme:
    the general kernel (taken because zero points are given) and the per-slot
    kernel agree bit for bit; so does the scheme call without zero points."""
    w = workloads.random_small(960, max_seqs=24, max_len=300, page_sizes=(16,), heads=(8,),
                               dims=(128,), dtypes=("i8",))
    say("per-block-affine == per-slot", w.describe())
    d = OnDevice(w)
    a = d.empty_out(dtype=torch.bfloat16)
    b = d.empty_out(dtype=torch.bfloat16)
    c = d.empty_out(dtype=torch.bfloat16)
    zeros = torch.zeros(w.num_pages * w.page_size, dtype=torch.int8, device=DEV)
    hp.gather_dequant(d.desc, a)
    hp.gather_dequant_q(d.desc, b, "per_block_affine", d.scales, zero_points=zeros)
    hp.gather_dequant_q(d.desc, c, "per_block_affine", d.scales)
    torch.cuda.synchronize()
    bf16_bits_equal(host_bits(b), host_bits(a), "per-block-affine (zero points) vs per-slot")
    bf16_bits_equal(host_bits(c), host_bits(a), "per-block-affine vs per-slot")


def test_rejected_scheme_writes_nothing(hp):
    """A scheme the layout rejects returns HP_ERR_QUANT and leaves out as it was."""
    w = workloads.random_small(970, max_seqs=8, max_len=50, page_sizes=(8,), heads=(2,),
                               dims=(16,), dtypes=("i8",))
    say("rejected scheme", w.describe())
    d = OnDevice(w)
    out = d.empty_out(dtype=torch.bfloat16)
    before = host_bits(out).copy()
    with pytest.raises(hp.HpError, match="HP_ERR_QUANT"):
        hp.gather_dequant_q(d.desc, out, "per_block_affine", d.scales, block_size=4)
    with pytest.raises(hp.HpError, match="HP_ERR_QUANT"):
        hp.gather_dequant_q(d.desc, out, "per_channel", d.scales, axis=0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), before)


def _subset(w, seqs):
    """Descriptor arrays of the sequences `seqs` only (same pool)."""
    sp = w.seq_ptr.astype(np.int64)
    bt = np.concatenate([w.block_table[sp[s]:sp[s + 1]] for s in seqs])
    counts = np.array([sp[s + 1] - sp[s] for s in seqs], dtype=np.int64)
    sub_sp = np.concatenate([[0], np.cumsum(counts)]).astype(w.seq_ptr.dtype)
    return bt, sub_sp, w.seq_lens[seqs]


@pytest.mark.parametrize("scheme,axis,with_zp", [("per_channel", 2, True),
                                                 ("per_channel", 1, False),
                                                 ("per_tensor", 0, True),
                                                 ("per_block_affine", 0, True)])
def test_scheme_full_quant_workload(hp, scheme, axis, with_zp):
    """1,024 log-normal sequences over the 200,000-page int8 pool: the whole
    output is produced in the launch shape the benchmark uses, and twelve
    sequences (the first, the last, the longest and nine at random) are
    compared with the oracle run on those sequences alone."""
    w = workloads.quant()
    say("dequant scheme full", scheme, axis, with_zp, w.describe())
    d = OnDevice(w)
    sc, zp = make_params(w, scheme, axis, 31, with_zp)
    sc_dev = torch.from_numpy(sc).to(DEV)
    zp_dev = None if zp is None else torch.from_numpy(zp).to(DEV)
    out = d.empty_out(dtype=torch.bfloat16)
    hp.gather_dequant_q(d.desc, out, scheme, sc_dev, axis=axis, zero_points=zp_dev)
    torch.cuda.synchronize()
    rng = np.random.default_rng(32)
    S = w.num_seqs
    seqs = sorted({0, S - 1, int(np.argmax(w.seq_lens))}
                  | set(rng.choice(S, size=9, replace=False).tolist()))
    bt, sp, sl = _subset(w, seqs)
    pool = host_bits(d.pool).view(np.int8)
    want = oracle.gather_dequant_scheme(pool, scheme, axis, sc, zp, page_size=w.page_size,
                                        num_heads=w.num_heads, head_dim=w.head_dim,
                                        block_table=bt, seq_ptr=sp, seq_lens=sl)
    tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    rows = np.concatenate([np.arange(tok[s], tok[s + 1]) for s in seqs])
    got = host_bits(out[torch.from_numpy(rows).to(DEV)])
    bf16_bits_equal(got, want, f"full {scheme} axis {axis}")
    del d, out
    torch.cuda.empty_cache()
