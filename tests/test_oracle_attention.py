"""Pins of the paged-attention oracle (CPU only).

The oracle computes decode attention over a block-paged K/V cache in binary64
([Day51] "How the attention kernel uses the block table"; [Rust20] "Keep token
order across cache pages": paging changes where rows live, not the dot
products). It is pinned here against things other than itself: the IEEE
decoders against numpy / torch conversions of every bit pattern, closed forms
(one token, equal keys, constant values, two tokens), torch's
scaled_dot_product_attention in float64 on the same rows gathered into a
contiguous tensor, a pure-Python brute force, the grouped-query head mapping,
relabelling of physical pages and shared prefix pages.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import brute

NP_BITS = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32}
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
TORCH_BITS = {"f16": torch.int16, "bf16": torch.int16, "f32": torch.int32}


def to_bits(t, dtype):
    return t.contiguous().view(TORCH_BITS[dtype]).numpy().view(NP_BITS[dtype])


def values(bits, dtype):
    """float64 values of stored bits through torch (a route independent of
    the oracle's decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if dtype != "f32" else np.int32))
    return t.view(TORCH[dtype]).to(torch.float64).numpy()


def case(seed, dtype="f16", group=1, heads=(1, 2, 3), dims=(1, 2, 4, 8, 16), max_seqs=5,
         max_len=40, page_sizes=(1, 2, 3, 4, 5, 8, 16), alias=True):
    """A random descriptor with K and V pools and queries, as bit patterns."""
    w = workloads.random_small(seed, max_seqs=max_seqs, max_len=max_len, page_sizes=page_sizes,
                               heads=heads, dims=dims, dtypes=(dtype,), alias=alias)
    g = torch.Generator().manual_seed(seed)
    shape = (w.num_pages, w.page_size, w.num_heads, w.head_dim)
    k = torch.randn(shape, generator=g).to(TORCH[dtype])
    v = torch.randn(shape, generator=g).to(TORCH[dtype])
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g).to(TORCH[dtype])
    return w, to_bits(q, dtype), to_bits(k, dtype), to_bits(v, dtype)


def run(w, q, k, v, dtype, scale=None):
    scale = 1.0 / math.sqrt(w.head_dim) if scale is None else scale
    return oracle.paged_attention(q, k, v, dtype, page_size=w.page_size,
                                  num_kv_heads=w.num_heads, head_dim=w.head_dim,
                                  block_table=w.block_table, seq_ptr=w.seq_ptr,
                                  seq_lens=w.seq_lens, scale=scale)


def slot_ids(w):
    """Flat slot index (phys * page_size + offset) of every logical row."""
    ids = []
    for s in range(w.num_seqs):
        for t in range(int(w.seq_lens[s])):
            phys = int(w.block_table[int(w.seq_ptr[s]) + t // w.page_size])
            ids.append(phys * w.page_size + t % w.page_size)
    return np.array(ids, dtype=np.int64)


# ---- the IEEE decoders -------------------------------------------------------

def test_decode_f16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_bf16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "bf16")
    want = values(bits, "bf16")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_f32_patterns():
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32),
                           np.array([0, 1, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x80000000,
                                     0x007FFFFF], dtype=np.uint32)])
    got = oracle.decode(bits, "f32")
    with np.errstate(invalid="ignore"):
        want = bits.view(np.float32).astype(np.float64)
    ok = ~np.isnan(want)
    assert np.array_equal(np.isnan(got), ~ok)
    assert np.array_equal(got[ok], want[ok])


# ---- closed forms -----------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_single_token_returns_its_value(dtype):
    """softmax over one token is 1: the output is that token's value row."""
    for seed in range(20):
        w, q, k, v = case(100 + seed, dtype, group=2)
        if not len(w.seq_lens):
            continue
        w.seq_lens[:] = np.minimum(w.seq_lens, 1)
        out = run(w, q, k, v, dtype)
        vals = values(v, dtype).reshape(-1, w.num_heads, w.head_dim)
        for s in range(w.num_seqs):
            for hq in range(out.shape[1]):
                if w.seq_lens[s] == 0:
                    assert np.all(out[s, hq] == 0)
                else:
                    phys = int(w.block_table[int(w.seq_ptr[s])])
                    assert np.array_equal(out[s, hq], vals[phys * w.page_size, hq // 2])


def test_equal_keys_average_the_values():
    """Identical keys give equal weights: the output is the mean of the value rows."""
    w, q, k, v = case(7, "f32", heads=(2,), dims=(8,), max_len=60)
    k[:] = k.reshape(-1, w.head_dim)[0].copy()          # every key row the same
    out = run(w, q, k, v, "f32")
    vals = values(v, "f32").reshape(-1, w.num_heads, w.head_dim)
    ids = slot_ids(w)
    tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    for s in range(w.num_seqs):
        if w.seq_lens[s]:
            rows = vals[ids[tok[s]:tok[s + 1]]]          # [L, Hkv, D]
            np.testing.assert_allclose(out[s], rows.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_constant_values_pass_through():
    """When every value row holds the same vector c, the output is c."""
    w, q, k, v = case(8, "bf16", heads=(3,), dims=(16,), max_len=80)
    c = to_bits(torch.linspace(-2, 2, w.head_dim).to(torch.bfloat16), "bf16")
    v[:] = np.broadcast_to(c, v.shape)
    out = run(w, q, k, v, "bf16")
    cv = values(c, "bf16")
    for s in range(w.num_seqs):
        if w.seq_lens[s]:
            np.testing.assert_allclose(out[s], np.broadcast_to(cv, out[s].shape), rtol=1e-14,
                                       atol=1e-15)


def test_two_tokens_logistic_weight():
    """Two tokens: the weight of token 0 is 1 / (1 + exp(x1 - x0))."""
    P, D = 4, 3
    q = np.array([[[1.0, 2.0, -1.0]]], dtype=np.float32).view(np.uint32)
    k = np.zeros((2, P, 1, D), dtype=np.float32)
    v = np.zeros((2, P, 1, D), dtype=np.float32)
    k[1, 0, 0] = [0.5, 0.25, 1.0]        # token 0 lives in page 1
    k[1, 1, 0] = [-1.0, 0.5, 2.0]        # token 1
    v[1, 0, 0] = [1.0, 0.0, 3.0]
    v[1, 1, 0] = [0.0, 1.0, -3.0]
    scale = 0.7
    out = oracle.paged_attention(q, k.view(np.uint32), v.view(np.uint32), "f32", page_size=P,
                                 num_kv_heads=1, head_dim=D, block_table=[1], seq_ptr=[0, 1],
                                 seq_lens=[2], scale=scale)
    x0 = scale * (0.5 * 1 + 0.25 * 2 + 1.0 * -1)
    x1 = scale * (-1.0 * 1 + 0.5 * 2 + 2.0 * -1)
    a = 1.0 / (1.0 + math.exp(x1 - x0))
    np.testing.assert_allclose(out[0, 0], [a, 1 - a, 3 * a - 3 * (1 - a)], rtol=1e-15,
                               atol=1e-16)


def test_empty_sequence_and_empty_batch():
    w, q, k, v = case(9, "f16", heads=(2,), dims=(4,))
    w.seq_lens[:] = 0
    assert np.all(run(w, q, k, v, "f16") == 0)
    out = oracle.paged_attention(np.zeros((0, 2, 4), np.uint16), k, v, "f16", page_size=w.page_size,
                                 num_kv_heads=2, head_dim=4, block_table=[], seq_ptr=[0],
                                 seq_lens=[], scale=0.5)
    assert out.shape == (0, 2, 4)


def test_rejects_query_heads_not_a_multiple():
    w, q, k, v = case(10, "f16", heads=(2,), dims=(4,))
    q3 = np.zeros((w.num_seqs, 3, 4), np.uint16)
    if w.num_seqs:
        with pytest.raises(ValueError):
            run(w, q3, k, v, "f16")


# ---- library and brute-force cross-checks ------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_sdpa_float64(seed, group, dtype):
    """torch's scaled_dot_product_attention in float64 on the sequence's rows
    gathered into a contiguous tensor, kv heads repeated for the groups."""
    w, q, k, v = case(200 + seed, dtype, group=group, max_len=70)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = run(w, q, k, v, dtype, scale)
    K = torch.from_numpy(values(k, dtype).reshape(-1, w.num_heads, w.head_dim))
    V = torch.from_numpy(values(v, dtype).reshape(-1, w.num_heads, w.head_dim))
    Q = torch.from_numpy(values(q, dtype))
    ids = torch.from_numpy(slot_ids(w))
    tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    for s in range(w.num_seqs):
        if w.seq_lens[s] == 0:
            continue
        rows = ids[tok[s]:tok[s + 1]]
        ks = K[rows].transpose(0, 1).repeat_interleave(group, dim=0).contiguous()  # [Hq, L, D]
        vs = V[rows].transpose(0, 1).repeat_interleave(group, dim=0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[s].unsqueeze(1).unsqueeze(0), ks.unsqueeze(0), vs.unsqueeze(0), scale=scale)
        np.testing.assert_allclose(out[s], ref[0, :, 0].numpy(), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed", range(25))
def test_matches_brute_force(seed):
    w, q, k, v = case(300 + seed, "f32", group=int(np.random.default_rng(seed).choice([1, 2, 3])),
                      heads=(1, 2), dims=(1, 2, 3, 5), max_seqs=4, max_len=20)
    scale = 0.3 + 0.1 * seed
    out = run(w, q, k, v, "f32", scale)
    shape = (w.num_pages, w.page_size, w.num_heads, w.head_dim)
    ref = brute.attention(values(q, "f32").tolist(), values(k, "f32").reshape(shape).tolist(),
                          values(v, "f32").reshape(shape).tolist(), w.block_table.tolist(),
                          w.seq_ptr.tolist(), w.seq_lens.tolist(), scale)
    if w.num_seqs:
        np.testing.assert_allclose(out, np.array(ref), rtol=1e-12, atol=1e-14)


def test_grouped_query_head_mapping():
    """Query head hq reads kv head hq // (Hq / Hkv): with one token and value
    rows that hold their kv-head index, output head hq is hq // group."""
    P, Hkv, D, group = 2, 3, 4, 4
    v = np.zeros((1, P, Hkv, D), dtype=np.float32)
    for j in range(Hkv):
        v[0, 0, j] = j
    k = np.ones((1, P, Hkv, D), dtype=np.float32)
    q = np.ones((1, Hkv * group, D), dtype=np.float32)
    out = oracle.paged_attention(q.view(np.uint32), k.view(np.uint32), v.view(np.uint32), "f32",
                                 page_size=P, num_kv_heads=Hkv, head_dim=D, block_table=[0],
                                 seq_ptr=[0, 1], seq_lens=[1], scale=1.0)
    for hq in range(Hkv * group):
        assert np.all(out[0, hq] == hq // group)


# ---- paging is storage only -------------------------------------------------

@pytest.mark.parametrize("seed", range(10))
def test_page_relabelling_changes_nothing(seed):
    """[Rust20]: where the pages live does not change the attention. Moving
    every page to a new physical ID (and the table with it) gives the same
    output, bit for bit."""
    w, q, k, v = case(400 + seed, "bf16", group=2, max_len=50)
    out = run(w, q, k, v, "bf16")
    perm = np.random.default_rng(seed).permutation(w.num_pages)   # old page i -> perm[i]
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm], v2[perm] = k, v
    w.block_table[:] = perm[w.block_table.astype(np.int64)].astype(w.block_table.dtype)
    assert np.array_equal(run(w, q, k2, v2, "bf16"), out)


def test_contiguous_storage_gives_the_same_result():
    """[Rust20]: the same rows stored in logical order (one page after
    another, identity table) give the paged result bit for bit."""
    w, q, k, v = case(450, "f16", group=2, max_len=60, alias=False)
    out = run(w, q, k, v, "f16")
    P = w.page_size
    kc = np.zeros_like(k)
    vc = np.zeros_like(v)
    pages = w.block_table.astype(np.int64)
    kc[: len(pages)] = k[pages]
    vc[: len(pages)] = v[pages]
    w2_bt = np.arange(len(pages), dtype=w.block_table.dtype)
    got = oracle.paged_attention(q, kc, vc, "f16", page_size=P, num_kv_heads=w.num_heads,
                                 head_dim=w.head_dim, block_table=w2_bt, seq_ptr=w.seq_ptr,
                                 seq_lens=w.seq_lens, scale=1.0 / math.sqrt(w.head_dim))
    assert np.array_equal(got, out)


def test_shared_prefix_pages():
    """[Hurray] Prefix Sharing: two sequences whose slices name the same pages
    (and have the same length and query) attend identically."""
    w, q, k, v = case(460, "f16", heads=(2,), dims=(8,), max_len=40)
    P = w.page_size
    bt = np.array([3, 1, 4, 3, 1, 4], dtype=np.uint32)
    sp = np.array([0, 3, 6], dtype=np.uint32)
    sl = np.array([min(3 * P, 7), min(3 * P, 7)], dtype=np.uint32)
    qq = np.stack([q[0], q[0]]) if len(q) else np.zeros((2, 2, 8), np.uint16)
    n = max(5, w.num_pages)
    kk = np.resize(k, (n,) + k.shape[1:]) if len(k) else np.zeros((n, P, 2, 8), np.uint16)
    vv = np.resize(v, (n,) + v.shape[1:]) if len(v) else np.zeros((n, P, 2, 8), np.uint16)
    out = oracle.paged_attention(qq, kk, vv, "f16", page_size=P, num_kv_heads=2, head_dim=8,
                                 block_table=bt, seq_ptr=sp, seq_lens=sl, scale=0.35)
    assert np.array_equal(out[0], out[1])
