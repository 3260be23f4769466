"""Calls every oracle entry point on small seeded descriptors, for the
sanitizer test (tests/test_oracle_sanitized.py), which runs this file in a
child process with an AddressSanitizer / UndefinedBehaviorSanitizer build of
the oracle loaded (HP_ORACLE_LIB) and the ASan runtime preloaded. Any report
aborts the child. Uses numpy only (no torch), so that nothing but the oracle
runs under the sanitizers' allocator. Not collected by pytest."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

assert oracle.LIB_PATH == os.environ.get("HP_ORACLE_LIB"), oracle.LIB_PATH


def pool_of(w, rng, dtype):
    shape = (w.num_pages, w.page_size, w.num_heads, w.head_dim)
    if dtype == np.int8:
        return rng.integers(-127, 128, size=shape, dtype=np.int8)
    if dtype == np.uint8:
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return rng.integers(0, 1 << 14, size=shape).astype(dtype)  # finite f16 / bf16 patterns


def kw(w):
    return dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)


calls = 0
for seed in range(60):
    rng = np.random.default_rng(9000 + seed)
    w = workloads.random_small(9000 + seed, max_seqs=6, max_len=40, with_start=seed % 2 == 0,
                               dtypes=("f16",))
    T = w.total_tokens
    v = oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages, page_size=w.page_size,
                        block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens,
                        total_tokens=T, seq_start=w.seq_start)
    assert v == ("valid", 0), v
    for zt in (False, True):
        oracle.disjoint_writes(num_pages=w.num_pages, page_size=w.page_size,
                               block_table=w.block_table, seq_ptr=w.seq_ptr,
                               seq_lens=w.seq_lens, seq_start=w.seq_start, zero_tail=zt)
    pool = pool_of(w, rng, np.uint16)
    out = oracle.gather(pool, **kw(w))
    _, mark = oracle.gather(pool, mark_reads=True, **kw(w))
    if T:
        oracle.gather_rows(pool, np.arange(T, dtype=np.uint64)[::3].copy(), **kw(w))
    src = rng.integers(0, 1 << 14, size=(T, w.num_heads, w.head_dim)).astype(np.uint16)
    for zt in (False, True):
        oracle.scatter(pool, src, seq_start=w.seq_start, zero_tail=zt, **kw(w))
    # int8 pool with per-slot scales
    qpool = pool_of(w, rng, np.int8)
    scales = rng.random(w.num_pages * w.page_size).astype(np.float32)
    oracle.gather_dequant(qpool, scales, **kw(w))
    if T:
        oracle.gather_dequant_rows(qpool, scales, np.arange(T, dtype=np.uint64)[::2].copy(),
                                   **kw(w))
    # other schemes, signed and unsigned
    upool = pool_of(w, rng, np.uint8)
    zp8 = rng.integers(0, 256, size=w.num_heads, dtype=np.uint8)
    oracle.gather_dequant_scheme(qpool, "per_tensor", 0, scales[:1].copy(), **kw(w))
    oracle.gather_dequant_scheme(upool, "per_channel", 1, scales[: w.num_heads].copy(), zp8,
                                 **kw(w))
    # copy-on-write page copies (distinct destinations)
    n = min(2, w.num_pages)
    srcp = np.arange(n, dtype=np.uint64)
    dstp = np.arange(w.num_pages - n, w.num_pages, dtype=np.uint64)
    if n and not set(srcp.tolist()) & set(dstp.tolist()):
        oracle.copy_pages(pool, srcp, dstp, page_size=w.page_size, num_heads=w.num_heads,
                          head_dim=w.head_dim, scales=scales)
    # quantize-on-scatter from f32 rows, both forms
    src32 = rng.standard_normal((T, w.num_heads, w.head_dim)).astype(np.float32)
    for asym in (False, True):
        p = upool if asym else qpool
        zp = np.zeros(w.num_pages * w.page_size, np.uint8) if asym else None
        oracle.scatter_quant(p, scales, src32.view(np.uint32), "f32", seq_start=w.seq_start,
                             zero_points=zp, zero_tail=True, **kw(w))
    # decode attention, two query heads per kv head
    G = 2
    q = rng.integers(0, 1 << 14, size=(w.num_seqs, w.num_heads * G, w.head_dim)).astype(np.uint16)
    oracle.paged_attention(q, pool, pool, "f16", page_size=w.page_size,
                           num_kv_heads=w.num_heads, head_dim=w.head_dim,
                           block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens,
                           scale=0.125)
    # the same over int8 pools with per-slot scales
    oracle.paged_attention_q8(q, qpool, scales, qpool, scales[::-1].copy(), page_size=w.page_size,
                              num_kv_heads=w.num_heads, head_dim=w.head_dim,
                              block_table=w.block_table, seq_ptr=w.seq_ptr,
                              seq_lens=w.seq_lens, scale=0.125)
    calls += 1
oracle.quantize_row(np.linspace(-3, 5, 33, dtype=np.float32), asym=True)
oracle.bf16_rne(np.linspace(-1, 1, 17, dtype=np.float32))
oracle.payload(capacity=64, page_tokens=16, length=40, batch=2, kv_heads=2, width=8)
print(f"sanitized oracle: {calls} descriptors, every entry point called", flush=True)
