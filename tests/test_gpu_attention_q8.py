"""GPU parity of decode attention over int8 K/V pools with one fp32 scale per
slot (hp_paged_attention_q8).

Every element's value is its code times its slot's scale ([Hurray]
Per-page-slot parameters). The kernels take the scale out of each token's
sums (x_t = scale sK_t q . c_t, weight p_t sV_t on the codes of V), which
changes only the fp32 rounding. Each case checks, on the same seeded inputs:

* against the oracle (binary64 over code * scale), with slot scales drawn
  from U[1e-3, 1e-1], within the fp32 bound of test_gpu_attention;
* with slot scales that are powers of two, bit for bit against
  hp_paged_attention over bf16 pools holding code * scale (which bf16 holds
  exactly, written by hp_gather_dequant): scaling by a power of two commutes
  with every rounding, so taking the scale out of the sums changes nothing.
  This holds where both calls split the work alike: on the matrix cores, and
  on the vector kernel with 8 codes per lane. With one or two query heads per
  kv head the vector kernel reads 16 codes per lane (a 16-byte load), so its
  lanes and token lanes differ from the 16-bit call's and its fp32 sums
  round in another order; there the oracle's bound is the check.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, assert_bits_equal, empty_seq_workload, host_bits, idx_tensor, say
from test_gpu_attention import shared_prefix_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def pow2_scales(n, seed):
    """Slot scales 2^-10 .. 2^-3, drawn per slot."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    e = torch.randint(-10, -2, (n,), generator=g, device=DEV)
    return torch.ldexp(torch.ones(n, device=DEV), e)


def int8_inputs(w, group, seed, pow2=False):
    """int8 K pool and K scales (the workload's), an int8 V pool and V scales
    from another seed, bf16 queries. pow2: power-of-two scales."""
    w = dataclasses.replace(w, dtype="i8", values="int8", with_scales=True)
    d = OnDevice(w)
    v = dataclasses.replace(w, seed=w.seed * 7 + 3)
    v_pool, v_scales = v.make_pool(DEV), v.make_scales(DEV)
    if pow2:
        n = w.num_pages * w.page_size
        d.scales.copy_(pow2_scales(n, seed + 1))
        v_scales = pow2_scales(n, seed + 2)
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g, device=DEV,
                    dtype=torch.float32).to(torch.bfloat16)
    return w, d, v_pool, v_scales, q


def run_q8(hp, w, d, v_pool, v_scales, q, scale, streaming=False):
    out = torch.full((w.num_seqs, q.shape[1], w.head_dim), float("nan"), device=DEV)
    hp.paged_attention_q8(d.desc, v_pool, v_scales, q, out, total_tokens=w.total_tokens,
                          scale=scale, streaming=streaming)
    torch.cuda.synchronize()
    return out


def dequant_pool(hp, pool, scales):
    """bf16 [N, P, H, D]: hp_gather_dequant of every slot (one sequence over
    pages 0..N-1)."""
    N, P, H, D = pool.shape
    ident = idx_tensor(np.arange(N, dtype=np.uint64), DEV)
    sp = idx_tensor(np.array([0, N], dtype=np.uint64), DEV)
    sl = idx_tensor(np.array([N * P], dtype=np.uint64), DEV)
    desc = hp.Descriptor(pool, ident, sp, sl, scales=scales)
    out = torch.empty((N * P, H, D), dtype=torch.bfloat16, device=DEV)
    hp.gather_dequant(desc, out)
    return out.view(N, P, H, D)


def slot_ids(w):
    out = []
    for s in range(w.num_seqs):
        base = int(w.seq_ptr[s])
        t = np.arange(int(w.seq_lens[s]), dtype=np.int64)
        phys = w.block_table[base + t // w.page_size].astype(np.int64)
        out.append(phys * w.page_size + t % w.page_size)
    return out


def tolerance(w, qv, kc, ks, vc, vs, scale, group):
    """The fp32 bound of test_gpu_attention per (sequence, query head), over
    the float64 values code * scale of the slots each sequence holds (codes
    kc, vc [slots, H, D], scales ks, vs [slots])."""
    heads = np.arange(qv.shape[1]) // group
    tol = np.zeros(qv.shape[:2])
    for i, ids in enumerate(slot_ids(w)):
        L = len(ids)
        if L == 0:
            continue
        Ks = (kc[ids].astype(np.float64) * ks[ids].astype(np.float64)[:, None, None])[:, heads, :]
        Vs = vc[ids].astype(np.float64) * vs[ids].astype(np.float64)[:, None, None]
        A = np.abs(scale * qv[i][None, :, :] * Ks).sum(axis=2).max(axis=0)
        vmax = np.abs(Vs).max(axis=(0, 2))[heads]
        delta = 2 * (w.head_dim + 16) * U * A + (3 * L + 16) * U
        tol[i] = 2.5 * delta * vmax
    return tol


def oracle_check(w, got, d, v_pool, v_scales, q, group, scale, what):
    H, D = w.num_heads, w.head_dim
    kc, vc = host_bits(d.pool).view(np.int8), host_bits(v_pool).view(np.int8)
    ks, vs = d.scales.cpu().numpy(), v_scales.cpu().numpy()
    qb = host_bits(q)
    want = oracle.paged_attention_q8(qb, kc, ks, vc, vs, page_size=w.page_size,
                                     num_kv_heads=H, head_dim=D, block_table=w.block_table,
                                     seq_ptr=w.seq_ptr, seq_lens=w.seq_lens, scale=scale)
    tol = tolerance(w, oracle.decode(qb, "bf16"), kc.reshape(-1, H, D), ks,
                    vc.reshape(-1, H, D), vs, scale, group)
    g = got.astype(np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN in the output"
    err = np.abs(g - want).max(axis=2) if g.size else np.zeros(tol.shape)
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    say(f"{what}: max error {float(err.max()) if err.size else 0:.3e}, "
        f"max error / bound {ratio:.3e}")
    bad = np.argwhere(err > tol)
    assert not len(bad), (f"{what}: {len(bad)} (seq, head) pairs over the bound; first "
                          f"{bad[:4].tolist()}")


def pow2_check(hp, w, d, v_pool, v_scales, q, scale, what, streaming=False):
    """Power-of-two scales: equal, bit for bit, to the 16-bit call over bf16
    pools holding code * scale."""
    out8 = run_q8(hp, w, d, v_pool, v_scales, q, scale, streaming)
    kb, vb = dequant_pool(hp, d.pool, d.scales), dequant_pool(hp, v_pool, v_scales)
    out16 = torch.full_like(out8, float("nan"))
    hp.paged_attention(hp.Descriptor(kb, d.bt, d.sp, d.sl), vb, q, out16,
                       total_tokens=w.total_tokens, scale=scale, streaming=streaming)
    torch.cuda.synchronize()
    assert_bits_equal(host_bits(out8), host_bits(out16), f"{what}: int8 call vs bf16 call")


def same_split(D, group, streaming):
    """Whether the int8 call splits its work as the 16-bit call does: the
    matrix-core kernel (head_dim 64 or 128 with three or more query heads per
    kv head, two with streaming loads), or the vector kernel with 8 codes per
    lane (head_dim 8, or more than two query heads per kv head)."""
    if D in (64, 128) and (group >= 3 or (streaming and group >= 2)):
        return True
    return D == 8 or group > 2


def both_checks(hp, w0, group, seed, scale, what, streaming=False):
    w, d, v_pool, v_scales, q = int8_inputs(w0, group, seed)
    out = run_q8(hp, w, d, v_pool, v_scales, q, scale, streaming)
    oracle_check(w, out.cpu().numpy(), d, v_pool, v_scales, q, group, scale, what)
    w, d, v_pool, v_scales, q = int8_inputs(w0, group, seed, pow2=True)
    if same_split(w.head_dim, group, streaming):
        pow2_check(hp, w, d, v_pool, v_scales, q, scale, what + " (power-of-two scales)",
                   streaming)
    else:
        out = run_q8(hp, w, d, v_pool, v_scales, q, scale, streaming)
        oracle_check(w, out.cpu().numpy(), d, v_pool, v_scales, q, group, scale,
                     what + " (power-of-two scales)")


CASES = [
    # (head_dim, group, kv heads, page sizes): vector kernel below G = 3 (or
    # head_dim other than 64 / 128), matrix cores from G = 3
    (128, 1, 8, (16,)),
    (128, 4, 8, (16,)),
    (64, 2, 4, (8, 16)),
    (256, 1, 2, (16, 32)),
    (32, 8, 1, (1, 3)),
    (16, 1, 20, (4,)),
    (8, 4, 3, (5,)),
    (128, 8, 2, (16,)),
    (64, 3, 6, (8, 16)),
    (128, 12, 2, (16,)),
    (128, 20, 2, (16,)),
    (64, 16, 4, (1, 3)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", range(2))
def test_attention_q8_random(hp, case, seed):
    D, group, hkv, pages = CASES[case]
    w = workloads.random_small(2100 + 10 * case + seed, max_seqs=12, max_len=300,
                               page_sizes=pages, heads=(hkv,), dims=(D,), dtypes=("i8",))
    say("attention int8", case, seed, group, w.describe())
    both_checks(hp, w, group, 2200 + 10 * case + seed, 1.0 / math.sqrt(D),
                what=f"int8 case {case} seed {seed}")


@pytest.mark.parametrize("group", [1, 2, 4])
def test_attention_q8_streaming(hp, group):
    """Streaming loads (the matrix cores from G = 2)."""
    w = workloads.random_small(2300 + group, max_seqs=12, max_len=400, page_sizes=(16,),
                               heads=(6,), dims=(128,), dtypes=("i8",), alias=False)
    say("attention int8 streaming", group, w.describe())
    both_checks(hp, w, group, 2310 + group, 0.09, what=f"int8 streaming G={group}",
                streaming=True)


@pytest.mark.parametrize("group", [1, 4])
def test_attention_q8_single_token_is_its_value_row(hp, group):
    """One cached token: its weight is 1, so the output is its value row,
    the fp32 product code * scale (bit for bit on the vector path at G = 1;
    within one ulp on the matrix cores at G = 4, which sum the weight's three
    bf16 parts)."""
    w = workloads.random_small(2320, max_seqs=16, max_len=40, page_sizes=(16,), heads=(4,),
                               dims=(128,), dtypes=("i8",))
    w.seq_lens[:] = np.minimum(w.seq_lens, 1)
    say("attention int8 single token", group, w.describe())
    w, d, v_pool, v_scales, q = int8_inputs(w, group, 2321 + group)
    out = run_q8(hp, w, d, v_pool, v_scales, q, 0.1).cpu().numpy()
    codes = host_bits(v_pool).view(np.int8).reshape(-1, 4, 128)
    sc = v_scales.cpu().numpy()
    for s in range(w.num_seqs):
        if w.seq_lens[s] == 0:
            assert np.all(out[s] == 0)
            continue
        row = int(w.block_table[int(w.seq_ptr[s])]) * w.page_size
        want = np.repeat(codes[row].astype(np.float32) * sc[row], group, axis=0)  # fp32 products
        if group == 1:
            assert np.array_equal(out[s], want), s
        else:
            ulp = np.spacing(np.abs(want))
            assert np.all(np.abs(out[s] - want) <= ulp), s


SHARED = [
    # (head_dim, G, kv heads, page size, index type, runs)
    (128, 4, 8, 16, np.uint32, [(12, 1024, (16, 300)), (1, 0, (5, 400)), (5, 512, (0, 40))]),
    (64, 8, 2, 16, np.uint64, [(7, 700, (1, 200)), (3, 64, (0, 0))]),
    (128, 32, 2, 16, np.uint32, [(3, 300, (1, 50)), (2, 48, (1, 50))]),
]


@pytest.mark.parametrize("case", range(len(SHARED)))
def test_attention_q8_shared_prefixes(hp, case):
    """Runs of sequences sharing leading pages: with cached loads the
    matrix-core grid carries the shared-prefix pass over the int8 pools."""
    D, G, H, P, idx, runs = SHARED[case]
    w = shared_prefix_workload(2400 + case, P, H, D, "i8", idx, runs)
    say("attention int8 shared prefixes", case, w.describe(), runs)
    both_checks(hp, w, G, 2410 + case, 1.0 / math.sqrt(D), what=f"int8 shared {case}")


def test_attention_q8_rejections(hp):
    w = workloads.random_small(2500, max_seqs=4, max_len=50, page_sizes=(16,), heads=(2,),
                               dims=(64,), dtypes=("i8",), num_seqs=3)
    w, d, v_pool, v_scales, q = int8_inputs(w, 2, 2501)
    out = torch.zeros((w.num_seqs, 4, 64), device=DEV)
    T = w.total_tokens
    with pytest.raises(hp.HpError, match="HP_ERR_NULL"):
        hp.paged_attention_q8(d.desc, v_pool, None, q, out, total_tokens=T)
    bare = hp.Descriptor(d.pool, d.bt, d.sp, d.sl)  # no K scales
    with pytest.raises(hp.HpError, match="HP_ERR_NULL"):
        hp.paged_attention_q8(bare, v_pool, v_scales, q, out, total_tokens=T)
    with pytest.raises(hp.HpError, match="HP_ERR_ALIGN"):
        hp.paged_attention_q8(d.desc, v_pool, v_scales[1:], q, out, total_tokens=T)
    # the output over the V scales: one buffer holds both
    n = v_scales.numel()
    buf = torch.zeros(n + out.numel(), device=DEV)
    buf[:n] = v_scales
    with pytest.raises(hp.HpError, match="HP_ERR_ARG"):
        hp.paged_attention_q8(d.desc, v_pool, buf[:n], q,
                              buf[n - 16: n - 16 + out.numel()].view(out.shape), total_tokens=T)
    # a bf16 pool is not an int8 pool (and the other way round)
    kb = torch.zeros(d.pool.shape, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(hp.HpError, match="HP_ERR_DTYPE"):
        hp.paged_attention_q8(hp.Descriptor(kb, d.bt, d.sp, d.sl), v_pool, v_scales, q, out,
                              total_tokens=T)
    with pytest.raises(hp.HpError, match="HP_ERR_DTYPE"):
        hp.paged_attention(d.desc, v_pool, q, out, total_tokens=T)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("group", [1, 4])
def test_attention_q8_decode_workload(hp, group):
    """The decode batch as int8 (64 sequences of 1..2048 tokens, 32 kv heads x
    128, per-slot scales) with one and four query heads per kv head and
    streaming loads, as the benchmark runs it: every sequence and query head
    against the oracle, and bit for bit against the 16-bit call with
    power-of-two scales."""
    w = workloads.decode()
    say("attention int8 decode full", group, w.describe())
    both_checks(hp, w, group, 2600 + group, 1.0 / math.sqrt(128), what=f"int8 decode G={group}",
                streaming=True)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("streaming", [False, True])
def test_attention_q8_empty_sequences_three_head_groups(hp, streaming):
    """Int8 pools on the matrix cores (G = 4) with three head groups (ten kv
    heads) and empty sequences first, last and between: head groups
    interleaved in the grid both streamed and cached."""
    w = empty_seq_workload("i8", 2500 + streaming)
    say("attention int8 empty sequences", streaming, w.describe())
    both_checks(hp, w, 4, 2510 + streaming, 1.0 / math.sqrt(w.head_dim),
                what=f"int8 empty sequences stream={streaming}", streaming=streaming)
