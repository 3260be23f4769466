"""GPU parity of decode attention over int8 K/V pools with one fp32 scale per
slot (hp_paged_attention_q8).

The call is defined as hp_paged_attention over bf16 pools that hold, in every
slot, the values hp_gather_dequant writes: bf16_rne(fp32(code) * scale). Each
case checks, on the same seeded inputs:

* the dequantized pools: hp_gather_dequant over an identity table (every slot
  of every page, in pool order) against the oracle's gather_dequant, bit for
  bit;
* the int8 call against hp_paged_attention over those bf16 pools, bit for
  bit (same units, same arithmetic);
* the int8 call against the oracle's attention (binary64) over the oracle's
  dequantized pools, within the fp32 bound of test_gpu_attention.
"""
import dataclasses
import math
import types

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, assert_bits_equal, host_bits, idx_tensor, say
from test_gpu_attention import check, shared_prefix_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def int8_inputs(w, group, seed):
    """int8 K pool and K scales (the workload's), an int8 V pool and V scales
    from another seed, bf16 queries."""
    w = dataclasses.replace(w, dtype="i8", values="int8", with_scales=True)
    d = OnDevice(w)
    v = dataclasses.replace(w, seed=w.seed * 7 + 3)
    v_pool, v_scales = v.make_pool(DEV), v.make_scales(DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g, device=DEV,
                    dtype=torch.float32).to(torch.bfloat16)
    return w, d, v_pool, v_scales, q


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


def oracle_dequant_pool(pool_bits, scales):
    N, P, H, D = pool_bits.shape
    return oracle.gather_dequant(pool_bits.view(np.int8), scales, page_size=P, num_heads=H,
                                 head_dim=D, block_table=np.arange(N, dtype=np.uint64),
                                 seq_ptr=np.array([0, N], dtype=np.uint64),
                                 seq_lens=np.array([N * P], dtype=np.uint64)).reshape(N, P, H, D)


def run_pair(hp, w, d, v_pool, v_scales, q, scale, streaming=False):
    """(int8 call, bf16 call over the dequantized pools, the bf16 pools)."""
    out8 = torch.full((w.num_seqs, q.shape[1], w.head_dim), float("nan"), device=DEV)
    hp.paged_attention_q8(d.desc, v_pool, v_scales, q, out8, total_tokens=w.total_tokens,
                          scale=scale, streaming=streaming)
    kb, vb = dequant_pool(hp, d.pool, d.scales), dequant_pool(hp, v_pool, v_scales)
    desc16 = hp.Descriptor(kb, d.bt, d.sp, d.sl)
    out16 = torch.full_like(out8, float("nan"))
    hp.paged_attention(desc16, vb, q, out16, total_tokens=w.total_tokens, scale=scale,
                       streaming=streaming)
    torch.cuda.synchronize()
    return out8, out16, kb, vb


def full_check(hp, w, d, v_pool, v_scales, q, group, scale, what, streaming=False,
               oracle_pools=True):
    out8, out16, kb, vb = run_pair(hp, w, d, v_pool, v_scales, q, scale, streaming)
    if oracle_pools:
        assert_bits_equal(host_bits(kb), oracle_dequant_pool(host_bits(d.pool),
                                                             d.scales.cpu().numpy()),
                          f"{what}: K pool dequantized")
        assert_bits_equal(host_bits(vb), oracle_dequant_pool(host_bits(v_pool),
                                                             v_scales.cpu().numpy()),
                          f"{what}: V pool dequantized")
    assert_bits_equal(host_bits(out8), host_bits(out16), f"{what}: int8 call vs bf16 call")
    w16 = dataclasses.replace(w, dtype="bf16", values="normal", with_scales=False)
    check(w16, out8.cpu().numpy(), q, types.SimpleNamespace(pool=kb), vb, group, scale,
          what=what)


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
    w, d, v_pool, v_scales, q = int8_inputs(w, group, 2200 + 10 * case + seed)
    full_check(hp, w, d, v_pool, v_scales, q, group, 1.0 / math.sqrt(D),
               what=f"int8 case {case} seed {seed}")


@pytest.mark.parametrize("group", [1, 2, 4])
def test_attention_q8_streaming(hp, group):
    """Streaming loads (the matrix cores from G = 2)."""
    w = workloads.random_small(2300 + group, max_seqs=12, max_len=400, page_sizes=(16,),
                               heads=(6,), dims=(128,), dtypes=("i8",), alias=False)
    say("attention int8 streaming", group, w.describe())
    w, d, v_pool, v_scales, q = int8_inputs(w, group, 2310 + group)
    full_check(hp, w, d, v_pool, v_scales, q, group, 0.09, streaming=True,
               what=f"int8 streaming G={group}")


def test_attention_q8_single_token_is_the_dequantized_row(hp):
    """One cached token: the output is its dequantized value row, bit for bit."""
    w = workloads.random_small(2320, max_seqs=16, max_len=40, page_sizes=(16,), heads=(4,),
                               dims=(128,), dtypes=("i8",))
    w.seq_lens[:] = np.minimum(w.seq_lens, 1)
    say("attention int8 single token", w.describe())
    for group in (1, 4):
        w, d, v_pool, v_scales, q = int8_inputs(w, group, 2321 + group)
        out = torch.zeros((w.num_seqs, 4 * group, 128), device=DEV)
        hp.paged_attention_q8(d.desc, v_pool, v_scales, q, out, total_tokens=w.total_tokens)
        torch.cuda.synchronize()
        vv = oracle.decode(oracle_dequant_pool(host_bits(v_pool), v_scales.cpu().numpy()),
                           "bf16").reshape(-1, 4, 128)
        got = out.cpu().numpy()
        for s in range(w.num_seqs):
            if w.seq_lens[s] == 0:
                assert np.all(got[s] == 0)
                continue
            row = int(w.block_table[int(w.seq_ptr[s])]) * w.page_size
            want = np.repeat(vv[row], group, axis=0)
            assert np.array_equal(got[s].astype(np.float64), want), (group, s)


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
    w, d, v_pool, v_scales, q = int8_inputs(w, G, 2410 + case)
    full_check(hp, w, d, v_pool, v_scales, q, G, 1.0 / math.sqrt(D),
               what=f"int8 shared {case}")


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


def test_attention_q8_decode_workload(hp):
    """The decode batch as int8 (64 sequences of 1..2048 tokens, 32 kv heads x
    128, per-slot scales) with four query heads per kv head and streaming
    loads: bit for bit against the bf16 call over the dequantized pools, and
    every sequence and query head against the oracle."""
    w = workloads.decode()
    say("attention int8 decode full", w.describe())
    w, d, v_pool, v_scales, q = int8_inputs(w, 4, 2600)
    full_check(hp, w, d, v_pool, v_scales, q, 4, 1.0 / math.sqrt(128), streaming=True,
               what="int8 decode", oracle_pools=False)
    del d, v_pool
    torch.cuda.empty_cache()
