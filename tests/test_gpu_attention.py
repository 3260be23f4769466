"""GPU parity of the decode attention over the block-paged K/V cache.

The HIP path (fp32 arithmetic, online softmax in base 2, units merged by a
combine kernel) is compared with the oracle (binary64) on the same seeded
inputs. The bound per (sequence, query head) follows from fp32 rounding:

* each score x_t = scale * q . k_t is off by at most E = (D + 16) u A, where
  A = max_t sum_d |scale q_d k_td| and u = 2^-24 (the dot product's D
  products and sums, the pre-scaled query, the base-2 conversion);
* the weights are then off by a factor within e^{+-E} relative to each
  other, and the exp2 evaluations, per-batch rescalings and fp32 sums over
  the L tokens add at most (3L + 16) u relative error;
* a convex combination of the value rows whose weights are perturbed by a
  relative delta moves by at most about 2 delta max|v|.

So |gpu - exact| <= 2.5 (2E + (3L + 16) u) max_t |v_t|, written in
`tolerance`. Structured cases check exact results where the arithmetic is
exact: one token gives its value row bit for bit; identical keys give equal
weights, so the output is the mean of the values.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import OnDevice, empty_seq_workload, host_bits, idx_tensor, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
U = 2.0 ** -24
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def _vals(bits, dtype):
    return oracle.decode(bits, dtype)


def make_inputs(w, group, seed, v_seed=None):
    """K pool (the workload's pool), a V pool of the same table and queries,
    all on the GPU from seeded generators."""
    d = OnDevice(w)
    v = dataclasses.replace(w, seed=w.seed * 7 + 3 if v_seed is None else v_seed)
    v_pool = v.make_pool(DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((w.num_seqs, w.num_heads * group, w.head_dim), generator=g, device=DEV,
                    dtype=torch.float32).to(TORCH[w.dtype])
    return d, v_pool, q


def slot_ids(w, seqs=None):
    """Flat slot index of every token of the listed sequences, per sequence."""
    out = []
    for s in (range(w.num_seqs) if seqs is None else seqs):
        base = int(w.seq_ptr[s])
        t = np.arange(int(w.seq_lens[s]), dtype=np.int64)
        phys = w.block_table[base + t // w.page_size].astype(np.int64)
        out.append(phys * w.page_size + t % w.page_size)
    return out


def tolerance(w, qv, k_bits, v_bits, scale, group, seqs):
    """Per (sequence, query head) bound of the module docstring. qv: float64
    [len(seqs), Hq, D]; k_bits, v_bits: the pools' bit patterns. Only the
    slots the listed sequences hold are decoded."""
    D, H = w.head_dim, w.num_heads
    k_rows = k_bits.reshape(-1, H * D)
    v_rows = v_bits.reshape(-1, H * D)
    heads = np.arange(qv.shape[1]) // group      # kv head of each query head
    tol = np.zeros(qv.shape[:2])
    for i, ids in enumerate(slot_ids(w, seqs)):
        L = len(ids)
        if L == 0:
            continue
        Ks = _vals(k_rows[ids], w.dtype).reshape(L, H, D)[:, heads, :]   # [L, Hq, D]
        Vs = _vals(v_rows[ids], w.dtype).reshape(L, H, D)
        A = np.abs(scale * qv[i][None, :, :] * Ks).sum(axis=2).max(axis=0)  # [Hq]
        vmax = np.abs(Vs).max(axis=(0, 2))[heads]                          # [Hq]
        delta = 2 * (D + 16) * U * A + (3 * L + 16) * U
        tol[i] = 2.5 * delta * vmax
    return tol


def oracle_attention(w, q_bits, k_bits, v_bits, scale, seqs=None):
    """The oracle on the listed sequences (each with its own slice of the
    table)."""
    if seqs is None:
        seqs = list(range(w.num_seqs))
    sp = w.seq_ptr.astype(np.int64)
    bt = (np.concatenate([w.block_table[sp[s]:sp[s + 1]] for s in seqs])
          if seqs else np.zeros(0, np.uint64))
    counts = [int(sp[s + 1] - sp[s]) for s in seqs]
    sub_sp = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint64)
    return oracle.paged_attention(q_bits[seqs], k_bits, v_bits, w.dtype, page_size=w.page_size,
                                  num_kv_heads=w.num_heads, head_dim=w.head_dim, block_table=bt,
                                  seq_ptr=sub_sp, seq_lens=w.seq_lens[seqs], scale=scale)


def check(w, got, q, d, v_pool, group, scale, seqs=None, what=""):
    seqs = list(range(w.num_seqs)) if seqs is None else seqs
    qb, kb, vb = host_bits(q), host_bits(d.pool), host_bits(v_pool)
    want = oracle_attention(w, qb, kb, vb, scale, seqs)
    tol = tolerance(w, _vals(qb[seqs], w.dtype), kb, vb, scale, group, seqs)
    g = got[seqs].astype(np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN in the output"
    err = np.abs(g - want).max(axis=2)
    ratio = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    say(f"{what}: max error {float(err.max()) if err.size else 0:.3e}, "
        f"max error / bound {ratio:.3e}")
    bad = np.argwhere(err > tol)
    assert not len(bad), (f"{what}: {len(bad)} (seq, head) pairs over the bound; first "
                          f"{bad[:4].tolist()} err {err[tuple(bad[0])]:.3e} "
                          f"tol {tol[tuple(bad[0])]:.3e}")


def run(hp, d, v_pool, q, w, scale, **kw):
    out = torch.full((w.num_seqs, q.shape[1], w.head_dim), float("nan"), device=DEV,
                     dtype=torch.float32)
    hp.paged_attention(d.desc, v_pool, q, out, total_tokens=w.total_tokens, scale=scale, **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # (dtype, head_dim, group, kv heads, page sizes)
    ("f16", 128, 1, 8, (16,)),
    ("bf16", 128, 4, 8, (16,)),
    ("f16", 64, 2, 4, (8, 16)),
    ("bf16", 256, 1, 2, (16, 32)),
    ("f16", 32, 8, 1, (1, 3)),
    ("bf16", 16, 1, 20, (4,)),
    ("f16", 8, 4, 3, (5,)),
    ("bf16", 128, 8, 2, (16,)),
    ("f16", 128, 2, 40, (16,)),        # 3 head groups, the last one partial
    ("bf16", 64, 1, 1, (2, 16)),       # one kv head: many token lanes
    ("f16", 256, 4, 5, (8,)),
    ("bf16", 8, 2, 64, (3,)),
    ("f16", 128, 3, 4, (16,)),         # group sizes that are not a power of two
    ("bf16", 64, 5, 2, (8,)),
    ("f16", 128, 7, 4, (16,)),
    ("bf16", 128, 12, 2, (16,)),       # more than 8 query heads per kv head: chunks of 8
    ("f16", 32, 16, 1, (4,)),
    # grouped heads on the matrix cores (G >= 3, head_dim 64 or 128)
    ("bf16", 128, 20, 2, (16,)),       # two row chunks of 16 query heads (16 + 4)
    ("f16", 64, 3, 6, (8, 16)),        # 4 + 2 kv heads: two idle waves in the last group
    ("bf16", 128, 4, 1, (16,)),        # one kv head: three idle waves
    ("f16", 128, 16, 4, (1, 3)),       # full 16 rows; 1- and 3-token pages inside a tile
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("seed", range(3))
def test_attention_random(hp, case, seed):
    dtype, D, group, hkv, pages = CASES[case]
    w = workloads.random_small(1100 + 10 * case + seed, max_seqs=12, max_len=300,
                               page_sizes=pages, heads=(hkv,), dims=(D,), dtypes=(dtype,))
    say("attention", case, seed, group, w.describe())
    d, v_pool, q = make_inputs(w, group, 1200 + case * 10 + seed)
    scale = 1.0 / math.sqrt(D)
    out = run(hp, d, v_pool, q, w, scale)
    check(w, out.cpu().numpy(), q, d, v_pool, group, scale, what=f"case {case} seed {seed}")


@pytest.mark.parametrize("group", [2, 4, 8])
def test_attention_single_token_is_exact(hp, group):
    """One cached token: its weight is exactly 1 and the output is its value
    row, bit for bit (vector path at G = 2, matrix cores at 4 and 8)."""
    w = workloads.random_small(1300, max_seqs=20, max_len=40, page_sizes=(16,), heads=(4,),
                               dims=(128,), dtypes=("bf16",))
    w.seq_lens[:] = np.minimum(w.seq_lens, 1)
    say("attention single token", group, w.describe())
    d, v_pool, q = make_inputs(w, group, 1301)
    out = run(hp, d, v_pool, q, w, 0.09).cpu().numpy()
    vv = _vals(host_bits(v_pool), "bf16").reshape(-1, w.num_heads, w.head_dim)
    for s in range(w.num_seqs):
        if w.seq_lens[s] == 0:
            assert np.all(out[s] == 0)
            continue
        row = int(w.block_table[int(w.seq_ptr[s])]) * w.page_size
        for hq in range(4 * group):
            got, want = out[s, hq].astype(np.float64), vv[row, hq // group]
            bad = np.flatnonzero(got != want)
            assert not len(bad), (f"seq {s} head {hq}: {len(bad)} differ, first {bad[:4]}: "
                                  f"got {got[bad[:4]]} want {want[bad[:4]]}")


@pytest.mark.parametrize("group", [1, 4])
def test_attention_equal_keys_give_the_mean(hp, group):
    """Identical keys: every weight is exactly 1, so the output is the mean of
    the value rows (fp32 sums of L terms; vector path at G = 1, matrix cores
    at G = 4)."""
    w = workloads.random_small(1310, max_seqs=10, max_len=500, page_sizes=(16,), heads=(8,),
                               dims=(128,), dtypes=("f16",))
    say("attention equal keys", group, w.describe())
    d, v_pool, q = make_inputs(w, group, 1311)
    g = torch.Generator(device=DEV).manual_seed(1312)
    krow = torch.randn(w.head_dim, generator=g, device=DEV).to(torch.float16)
    d.pool.copy_(krow.expand_as(d.pool))
    out = run(hp, d, v_pool, q, w, 0.1).cpu().numpy()
    vv = _vals(host_bits(v_pool), "f16").reshape(-1, w.num_heads, w.head_dim)
    for s, ids in enumerate(slot_ids(w)):
        if len(ids):
            mean = vv[ids].mean(axis=0)  # [H, D]; query head hq reads kv head hq // group
            bound = (2 * len(ids) + 8) * U * np.abs(vv[ids]).max()
            got = out[s].reshape(w.num_heads, group, w.head_dim)
            assert np.abs(got - mean[:, None, :]).max() <= bound


def test_attention_constant_values(hp):
    """Every value row the same vector c: the output is c up to the rounding
    of sum_t p_t c / sum_t p_t."""
    w = workloads.random_small(1320, max_seqs=10, max_len=500, page_sizes=(8,), heads=(2,),
                               dims=(64,), dtypes=("bf16",))
    say("attention constant values", w.describe())
    d, v_pool, q = make_inputs(w, 4, 1321)
    c = torch.linspace(-3, 3, 64, device=DEV).to(torch.bfloat16)
    v_pool.copy_(c.expand_as(v_pool))
    out = run(hp, d, v_pool, q, w, 0.125).cpu().numpy()
    cv = c.float().cpu().numpy().astype(np.float64)
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        if L:
            assert np.abs(out[s] - cv).max() <= (4 * L + 16) * U * 3.0


def test_attention_streaming_and_repeat_are_bit_identical(hp):
    w = workloads.random_small(1330, max_seqs=12, max_len=300, page_sizes=(16,), heads=(8,),
                               dims=(128,), dtypes=("f16",), alias=False)
    say("attention streaming", w.describe())
    d, v_pool, q = make_inputs(w, 4, 1331)
    a = run(hp, d, v_pool, q, w, 0.088)
    b = run(hp, d, v_pool, q, w, 0.088, streaming=True)
    c = run(hp, d, v_pool, q, w, 0.088)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


@pytest.mark.parametrize("D", [64, 128])
def test_attention_g2_streaming_and_cached(hp, D):
    """Two query heads per kv head: with streaming loads the matrix-core kernel
    runs, without them the vector kernel; both against the oracle."""
    w = workloads.random_small(1335 + D, max_seqs=12, max_len=400, page_sizes=(16,), heads=(6,),
                               dims=(D,), dtypes=("bf16",), alias=False)
    say("attention G=2 streaming and cached", D, w.describe())
    d, v_pool, q = make_inputs(w, 2, 1336 + D)
    for streaming in (True, False):
        out = run(hp, d, v_pool, q, w, 0.09, streaming=streaming).cpu().numpy()
        check(w, out, q, d, v_pool, 2, 0.09, what=f"G=2 D={D} streaming={streaming}")


def test_attention_empty_and_short_sequences(hp):
    """Sequences of 0..3 tokens next to long ones; one kv head, so most lane
    groups of a workgroup are token lanes that see no token."""
    rng = np.random.default_rng(1340)
    lens = np.array([0, 1, 2, 3, 0, 700, 1, 0, 33], dtype=np.uint32)
    P = 16
    counts = (lens + P - 1) // P
    K = int(counts.sum())
    bt = rng.permutation(K + 5)[:K].astype(np.uint32)
    sp = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    w = workloads.Workload("short", "bf16", P, 1, 128, K + 5, np.uint32, bt, sp, lens, seed=1340)
    say("attention short", w.describe())
    d, v_pool, q = make_inputs(w, 8, 1341)
    out = run(hp, d, v_pool, q, w, 0.088)
    res = out.cpu().numpy()
    assert np.all(res[lens == 0] == 0)
    check(w, res, q, d, v_pool, 8, 0.088, what="short")


def test_attention_many_sequences_plan_path(hp):
    """More sequences than the attention kernels count themselves: the plan
    kernel writes the unit table and the unit -> sequence map."""
    rng = np.random.default_rng(1360)
    S, P = 4600, 4
    lens = rng.integers(0, 24, size=S).astype(np.uint32)
    counts = (lens + P - 1) // P
    K = int(counts.sum())
    bt = rng.permutation(K + 7)[:K].astype(np.uint32)
    sp = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    w = workloads.Workload("plan", "bf16", P, 2, 64, K + 7, np.uint32, bt, sp, lens, seed=1360)
    say("attention plan path", w.describe())
    d, v_pool, q = make_inputs(w, 2, 1361)
    out = run(hp, d, v_pool, q, w, 0.125).cpu().numpy()
    assert np.all(out[lens == 0] == 0)
    check(w, out, q, d, v_pool, 2, 0.125, what="plan path")


def test_attention_checked_rejects_bad_table(hp):
    w = workloads.random_small(1350, max_seqs=6, max_len=60, page_sizes=(16,), heads=(2,),
                               dims=(64,), dtypes=("f16",))
    while len(w.block_table) == 0:
        w = workloads.random_small(int(w.seed) + 1, max_seqs=6, max_len=60, page_sizes=(16,),
                                   heads=(2,), dims=(64,), dtypes=("f16",))
    say("attention checked", w.describe())
    d, v_pool, q = make_inputs(w, 1, 1351)
    bad = w.block_table.copy()
    bad[-1] = w.num_pages                       # one page ID past the pool
    bt = idx_tensor(bad.astype(w.index_dtype), DEV)
    desc = hp.Descriptor(d.pool, bt, d.sp, d.sl)
    out = torch.zeros((w.num_seqs, 2, 64), device=DEV)
    with pytest.raises(hp.HpError, match="HP_ERR_PAGE_RANGE"):
        hp.paged_attention(desc, v_pool, q, out, total_tokens=w.total_tokens, checked=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_attention_decode_workload(hp):
    """64 sequences of 1..2048 tokens, 32 kv heads x 128 fp16 (one query head
    per kv head), in the launch shape the benchmark uses (streaming loads);
    every sequence and query head against the oracle."""
    w = workloads.decode()
    say("attention decode full", w.describe())
    d, v_pool, q = make_inputs(w, 1, 1400)
    scale = 1.0 / math.sqrt(128)
    out = run(hp, d, v_pool, q, w, scale, streaming=True).cpu().numpy()
    check(w, out, q, d, v_pool, 1, scale, what="decode")
    del d, v_pool
    torch.cuda.empty_cache()


def test_attention_prefix_workload_gqa(hp):
    """256 sequences sharing 64 prefix pages, 8 kv heads x 128 bf16 and 32
    query heads (groups of 4); cached loads, since the prefix pages are read
    by every sequence. Every sequence and query head against the oracle."""
    w = workloads.prefix()
    say("attention prefix full", w.describe())
    d, v_pool, q = make_inputs(w, 4, 1410)
    scale = 1.0 / math.sqrt(128)
    out = run(hp, d, v_pool, q, w, scale).cpu().numpy()
    check(w, out, q, d, v_pool, 4, scale, what="prefix")
    del d, v_pool
    torch.cuda.empty_cache()


def test_attention_pools_beyond_4gib(hp):
    """K and V pools of 150,000 pages x 16 x 8 x 128 bf16 (4.9 GB each) with a
    uint64 table whose pages lie mostly past the 4 GiB byte offset: 64-bit row
    offsets, 24 sequences against the oracle."""
    rng = np.random.default_rng(1500)
    N, P, H, D = 150_000, 16, 8, 128
    lens = rng.integers(1, 700, size=24)
    counts = (lens + P - 1) // P
    high = rng.permutation(np.arange(140_000, N))[: int(counts.sum())]
    high[::5] = rng.integers(0, 500, size=len(high[::5]))  # a few low pages too
    w = workloads.Workload("pool5g", "bf16", P, H, D, N, np.uint64, high.astype(np.uint64),
                           np.concatenate([[0], np.cumsum(counts)]).astype(np.uint64),
                           lens.astype(np.uint64), seed=1500)
    say("attention pools > 4 GiB", w.describe())
    d, v_pool, q = make_inputs(w, 4, 1501)
    out = run(hp, d, v_pool, q, w, 0.088, streaming=True).cpu().numpy()
    check(w, out, q, d, v_pool, 4, 0.088, what="pools > 4 GiB")
    del d, v_pool
    torch.cuda.empty_cache()


# ---- shared prefixes (the shared-prefix pass) ---------------------------------------------

def shared_prefix_workload(seed, P, H, D, dtype, idx, runs):
    """Runs of sequences whose slices begin with the same pages. runs: a list
    of (sequences in the run, shared tokens, (min, max) suffix tokens); a run
    of one is an unshared sequence. The shared tokens need not fill whole
    pages: a partial last shared page is the run members' own page (copies of
    the shared page's tokens are not needed: different pages, different
    values). Pages are numbered in order of use, then permuted over the pool
    (which holds exactly the pages used plus three spares)."""
    rng = np.random.default_rng(seed)
    slices, lens = [], []
    nxt = 0
    for n_seq, shared_tok, (lo, hi) in runs:
        full = shared_tok // P
        shared_pages = np.arange(nxt, nxt + full)
        nxt += full
        for _ in range(n_seq):
            L = shared_tok + int(rng.integers(lo, hi + 1))
            own = (L - full * P + P - 1) // P
            slices.append(np.concatenate([shared_pages, np.arange(nxt, nxt + own)]))
            nxt += own
            lens.append(L)
    num_pages = nxt + 3
    perm = rng.permutation(num_pages)
    bt = perm[np.concatenate(slices)].astype(idx)
    sp = np.concatenate([[0], np.cumsum([len(x) for x in slices])]).astype(idx)
    return workloads.Workload("shared", dtype, P, H, D, num_pages, idx, bt, sp,
                              np.array(lens, dtype=idx), seed=seed)


SHARED_CASES = [
    # (dtype, head_dim, G, kv heads, page size, index type, runs)
    ("bf16", 128, 4, 8, 16, np.uint32, [(12, 1024, (16, 300)), (1, 0, (5, 400)), (5, 512, (0, 40))]),
    ("f16", 128, 8, 2, 16, np.uint64, [(7, 700, (1, 200)), (3, 64, (0, 0)), (1, 0, (1, 90))]),
    ("bf16", 64, 3, 4, 8, np.uint32, [(11, 333, (0, 100)), (2, 256, (30, 30))]),
    ("f16", 64, 16, 1, 16, np.uint32, [(3, 256, (0, 0)), (4, 1000, (1, 64))]),   # one sequence per block
    ("bf16", 128, 32, 2, 16, np.uint64, [(3, 300, (1, 50)), (2, 48, (1, 50))]),   # G > 16; a run below 64 tokens
    ("f16", 64, 5, 3, 5, np.uint32, [(9, 400, (0, 33)), (1, 0, (1, 1))]),         # odd page size
    ("bf16", 128, 4, 4, 16, np.uint32, [(40, 2048, (1, 16))]),                    # long shared part, 8 chunks
    ("f16", 64, 4, 1, 1, np.uint32, [(3, 9000, (0, 20)), (2, 100, (3, 9))]),      # 9,000 shared pages: past the comparison cap
    ("bf16", 64, 4, 1, 16, np.uint32, [(100, 64, (0, 8))] * 26),                  # 2,600 sequences: the plan's arrays in the workspace
]


@pytest.mark.parametrize("case", range(len(SHARED_CASES)))
def test_attention_shared_prefixes(hp, case):
    """Sequences in runs that share leading pages: with cached loads the
    matrix-core path computes each run's shared part once per kv head and
    chunk for several sequences at a time, the suffixes per sequence, and
    merges them. Every sequence and query head against the oracle; the
    streaming hint (which skips the shared pass) must give the same answer
    within the same bound."""
    dtype, D, G, H, P, idx, runs = SHARED_CASES[case]
    w = shared_prefix_workload(1600 + case, P, H, D, dtype, idx, runs)
    say("attention shared prefixes", case, w.describe(), runs)
    d, v_pool, q = make_inputs(w, G, 1601 + case)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    scale = 1.0 / math.sqrt(D)
    out = run(hp, d, v_pool, q, w, scale).cpu().numpy()
    check(w, out, q, d, v_pool, G, scale, what=f"shared {case}")
    out_nt = run(hp, d, v_pool, q, w, scale, streaming=True).cpu().numpy()
    check(w, out_nt, q, d, v_pool, G, scale, what=f"shared {case}, streamed")


def test_attention_shared_exact_cases(hp):
    """A shared part with one token's key repeated: every sequence of the run
    whose suffix is empty and whose shared part holds identical keys gets the
    mean of the shared values; a sequence held entirely by one shared chunk
    is written by the shared pass directly."""
    P, H, D, G = 16, 2, 64, 4
    w = shared_prefix_workload(1650, P, H, D, "bf16", np.uint32, [(6, 128, (0, 0))])
    say("attention shared exact", w.describe())
    d, v_pool, q = make_inputs(w, G, 1651)
    assert hp.validate(d.desc, w.total_tokens) == ("HP_OK", 0)
    # identical keys on the shared pages: equal weights, so each output is the
    # mean of the shared values
    ids = np.unique(w.block_table.astype(np.int64))
    kp = d.pool.view(torch.int16)
    first = kp[int(ids[0]), 0].clone()
    kp[torch.from_numpy(ids).to(DEV)] = first
    torch.cuda.synchronize()
    out = run(hp, d, v_pool, q, w, 0.2).cpu().numpy()
    vals = _vals(host_bits(v_pool), "bf16").reshape(-1, H, D)
    slots = slot_ids(w, [0])[0]
    mean = vals[slots].mean(axis=0)  # [H, D]
    # every weight is exactly 1: fp32 sums of L terms, then one division
    bound = (2 * len(slots) + 8) * U * np.abs(vals[slots]).max()
    got = out.reshape(w.num_seqs, H, G, D)
    assert np.abs(got - mean[None, :, None, :]).max() <= bound


@pytest.mark.parametrize("streaming", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_empty_sequences_three_head_groups(hp, dtype, streaming):
    """Matrix-core grids (G = 4) with three head groups and empty sequences:
    every head of an empty sequence is written as zeros (the output starts as
    NaN), streamed (head groups interleaved in the grid) and cached (the grid
    that carries the shared-prefix pass)."""
    w = empty_seq_workload(dtype, 1500 + streaming)
    say("attention empty sequences", dtype, streaming, w.describe())
    d, v_pool, q = make_inputs(w, 4, 1510 + streaming)
    scale = 1.0 / math.sqrt(w.head_dim)
    out = run(hp, d, v_pool, q, w, scale, streaming=streaming)
    got = out.cpu().numpy()
    for s in np.flatnonzero(w.seq_lens == 0):
        assert np.all(got[s] == 0), f"sequence {s}"
    check(w, got, q, d, v_pool, 4, scale, what=f"empty sequences {dtype} stream={streaming}")
