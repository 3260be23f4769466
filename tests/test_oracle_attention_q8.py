"""Pins of the paged-attention oracle over int8 K/V pools with one float32
scale per physical slot (CPU only).

[Hurray] Per-page-slot parameters: the value of every element of a slot's
row is its code times the slot's scale, the scale of slot r of page p being
scales[p * page_size + r]. The oracle attends over those values in binary64
(the products are exact there). It is pinned against: the 16-bit oracle on
bf16 pools that hold the codes (unit scales), torch's
scaled_dot_product_attention in float64 on the dequantized rows gathered
into a contiguous tensor, a pure-Python brute force, and per-slot edits
(a zero K scale is a zeroed K row; a doubled V scale is doubled V codes).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import brute


def case(seed, group=1, heads=(1, 2, 3), dims=(1, 2, 4, 8, 16), max_seqs=5, max_len=40,
         page_sizes=(1, 2, 3, 4, 5, 8, 16), code_max=127):
    """A random descriptor with int8 K and V pools, their slot scales and bf16
    queries (as bit patterns)."""
    w = workloads.random_small(seed, max_seqs=max_seqs, max_len=max_len, page_sizes=page_sizes,
                               heads=heads, dims=dims, dtypes=("i8",))
    rng = np.random.default_rng(seed)
    shape = (w.num_pages, w.page_size, w.num_heads, w.head_dim)
    k = rng.integers(-code_max, code_max + 1, size=shape).astype(np.int8)
    v = rng.integers(-code_max, code_max + 1, size=shape).astype(np.int8)
    ks = (rng.random(w.num_pages * w.page_size) * (1e-1 - 1e-3) + 1e-3).astype(np.float32)
    vs = (rng.random(w.num_pages * w.page_size) * (1e-1 - 1e-3) + 1e-3).astype(np.float32)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g)
    qb = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return w, qb, k, ks, v, vs


def run(w, q, k, ks, v, vs, scale):
    return oracle.paged_attention_q8(q, k, ks, v, vs, page_size=w.page_size,
                                     num_kv_heads=w.num_heads, head_dim=w.head_dim,
                                     block_table=w.block_table, seq_ptr=w.seq_ptr,
                                     seq_lens=w.seq_lens, scale=scale)


def bf16_values(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def slot_ids(w):
    ids = []
    for s in range(w.num_seqs):
        for t in range(int(w.seq_lens[s])):
            phys = int(w.block_table[int(w.seq_ptr[s]) + t // w.page_size])
            ids.append(phys * w.page_size + t % w.page_size)
    return np.array(ids, dtype=np.int64)


@pytest.mark.parametrize("seed", range(10))
def test_unit_scales_equal_the_16bit_oracle_on_the_codes(seed):
    """Scales of 1: the values are the codes, which bf16 holds exactly, so the
    result equals the 16-bit oracle's on bf16 pools of the codes, bit for bit
    (the same binary64 operations in the same order)."""
    w, q, k, _, v, _ = case(3000 + seed, group=1 + seed % 3)
    ones = np.ones(w.num_pages * w.page_size, np.float32)
    got = run(w, q, k, ones, v, ones, 0.37)
    to_bf16 = lambda c: (torch.from_numpy(c.astype(np.float32)).to(torch.bfloat16)
                         .view(torch.int16).numpy().view(np.uint16))
    want = oracle.paged_attention(q, to_bf16(k), to_bf16(v), "bf16", page_size=w.page_size,
                                  num_kv_heads=w.num_heads, head_dim=w.head_dim,
                                  block_table=w.block_table, seq_ptr=w.seq_ptr,
                                  seq_lens=w.seq_lens, scale=0.37)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("group", [1, 2, 4])
@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_sdpa_float64(seed, group):
    """torch's scaled_dot_product_attention in float64 on the rows gathered
    through the table and dequantized by torch (code * scale of the row's
    slot), kv heads repeated for the groups."""
    w, q, k, ks, v, vs = case(3100 + seed, group=group, max_len=70)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = run(w, q, k, ks, v, vs, scale)
    H, D = w.num_heads, w.head_dim
    K = torch.from_numpy(k.reshape(-1, H, D)).double() * torch.from_numpy(ks).double()[:, None, None]
    V = torch.from_numpy(v.reshape(-1, H, D)).double() * torch.from_numpy(vs).double()[:, None, None]
    Q = torch.from_numpy(bf16_values(q))
    ids = torch.from_numpy(slot_ids(w))
    tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])
    for s in range(w.num_seqs):
        if w.seq_lens[s] == 0:
            assert np.all(out[s] == 0)
            continue
        rows = ids[tok[s]:tok[s + 1]]
        kk = K[rows].transpose(0, 1).repeat_interleave(group, dim=0).contiguous()  # [Hq, L, D]
        vv = V[rows].transpose(0, 1).repeat_interleave(group, dim=0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q[s].unsqueeze(1).unsqueeze(0), kk.unsqueeze(0), vv.unsqueeze(0), scale=scale)
        np.testing.assert_allclose(out[s], ref[0, :, 0].numpy(), rtol=1e-11, atol=1e-15)


@pytest.mark.parametrize("seed", range(15))
def test_matches_brute_force(seed):
    w, q, k, ks, v, vs = case(3200 + seed, group=1 + seed % 2, heads=(1, 2), dims=(1, 2, 3, 5),
                              max_seqs=4, max_len=20)
    scale = 0.3 + 0.1 * seed
    out = run(w, q, k, ks, v, vs, scale)
    P, H, D = w.page_size, w.num_heads, w.head_dim
    shape = (w.num_pages, P, H, D)
    slot_scale = lambda sc: np.repeat(sc.astype(np.float64), H * D).reshape(shape)
    kv = (k.astype(np.float64) * slot_scale(ks)).tolist()
    vv = (v.astype(np.float64) * slot_scale(vs)).tolist()
    ref = brute.attention(bf16_values(q).tolist(), kv, vv, w.block_table.tolist(),
                          w.seq_ptr.tolist(), w.seq_lens.tolist(), scale)
    if w.num_seqs:
        np.testing.assert_allclose(out, np.array(ref), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_scales_belong_to_their_slot(seed):
    """A zero K scale on one slot gives what zeroed K codes on that slot give;
    a doubled V scale on one slot gives what doubled V codes give (codes in
    [-63, 63], so doubling stays in range and every product is exact)."""
    w, q, k, ks, v, vs = case(3300 + seed, group=2, max_len=60, code_max=63)
    ids = slot_ids(w)
    if not len(ids):
        pytest.skip("empty batch")
    slot = int(ids[len(ids) // 2])
    k2, ks2 = k.reshape(-1, w.num_heads, w.head_dim).copy(), ks.copy()
    ks2[slot] = 0.0
    k3 = k2.copy()
    k3[slot] = 0
    a = run(w, q, k2.reshape(k.shape), ks2, v, vs, 0.25)
    b = run(w, q, k3.reshape(k.shape), ks, v, vs, 0.25)
    assert np.array_equal(a, b)
    vs2 = vs.copy()
    vs2[slot] *= 2.0
    v3 = v.reshape(-1, w.num_heads, w.head_dim).copy()
    v3[slot] *= 2
    a = run(w, q, k, ks, v, vs2, 0.25)
    b = run(w, q, k, ks, v3.reshape(v.shape), vs, 0.25)
    assert np.array_equal(a, b)
    # and the edit changes the sequences that hold the slot
    c = run(w, q, k, ks, v, vs, 0.25)
    assert not np.array_equal(a, c)
