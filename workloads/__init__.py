"""Seeded synthetic inputs for the block-paged gather/scatter path.

This module only builds inputs: sequence lengths, block tables, seq_ptr
offsets and pool/source/scale values. It holds none of the path's arithmetic
(no element lookup, no copy, no dequantisation), and it is the only code that
both the GPU tests/benchmark and the CPU oracle consume.

Structure (lengths, tables) comes from numpy PCG64 with a fixed seed per
workload, so it is identical on every machine. Element values come from a
seeded torch.Generator on the device the caller names (values drawn on the
GPU for the large pools, since drawing gigabytes on the host takes minutes);
the oracle then reads a host copy of exactly those bytes.

Shapes follow the pages' examples:

* tiny: [Day51] "Visualizing the layout" (three requests of 40, 24 and 50
  tokens in a 20-block pool with 16-token blocks);
* decode: [Day51] "The block abstraction" (block size 16, 32 heads x 128,
  fp16) with the pool sized for one layer;
* prefix: [Hurray] "Prefix Sharing" (slices that alias leading pages);
* append: [Day51] RequestState.append_token (one new token per decode step)
  and [Hurray] "Partial trailing page" (writer zeroes unused slots);
* quant: [Hurray] "Per-page-slot parameters" (one fp32 scale per slot).
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Storage dtypes the library moves, with their element widths in bytes.
DTYPE_BYTES = {"i8": 1, "u8": 1, "f16": 2, "bf16": 2, "f32": 4, "f64": 8}

# Bit pattern written into pool slots that no sequence references (a NaN with
# a payload for the floating types, so that a copied sentinel is recognisable).
SENTINEL_BITS = {1: 0x5A, 2: 0x7E5A, 4: 0x7FC05A5A, 8: 0x7FF85A5A5A5A5A5A}


def torch_dtype(name):
    import torch
    return {"i8": torch.int8, "u8": torch.uint8, "f16": torch.float16,
            "bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[name]


def bits_dtype(nbytes):
    """Integer torch dtype of the same width (for bit-exact comparisons)."""
    import torch
    return {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[nbytes]


def np_bits_dtype(nbytes):
    return {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[nbytes]


@dataclass
class Workload:
    """One block-paged descriptor plus the recipe for its element values."""
    name: str
    dtype: str
    page_size: int
    num_heads: int
    head_dim: int
    num_pages: int
    index_dtype: type
    block_table: np.ndarray
    seq_ptr: np.ndarray
    seq_lens: np.ndarray
    seq_start: Optional[np.ndarray] = None
    zero_tail: bool = False
    values: str = "normal"           # "normal", "uniform1" (U[-1,1]) or "int8"
    with_scales: bool = False         # per-slot fp32 scales U[1e-3, 1e-1]
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.seq_lens)

    @property
    def total_tokens(self):
        return int(self.seq_lens.sum()) if len(self.seq_lens) else 0

    @property
    def num_block_entries(self):
        return len(self.block_table)

    @property
    def elem_bytes(self):
        return DTYPE_BYTES[self.dtype]

    @property
    def row_bytes(self):
        return self.num_heads * self.head_dim * self.elem_bytes

    def referenced_pages(self):
        """Page IDs the block table names that exist in the pool (IDs out of
        range, as in deliberately invalid descriptors, are skipped)."""
        ids = np.unique(self.block_table.astype(np.int64))
        return ids[(ids >= 0) & (ids < self.num_pages)]

    # ---- element values (seeded, on any torch device) -------------------
    def _generator(self, device, salt):
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(self.seed * 1000 + salt)
        return g

    def _values(self, shape, device, gen):
        import torch
        if self.values == "int8":
            return torch.randint(-127, 128, shape, generator=gen, device=device,
                                 dtype=torch.int8)
        dt = torch_dtype(self.dtype)
        if self.values == "uniform1":
            x = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
            return (x * 2.0 - 1.0).to(dt)
        if dt in (torch.int8, torch.uint8):
            return torch.randint(0, 256, shape, generator=gen, device=device,
                                 dtype=torch.int16).to(dt)
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dt)

    def make_pool(self, device="cpu"):
        """[num_pages, P, H, D] pool: random values in every referenced page,
        the sentinel bit pattern in every other page."""
        import torch
        shape = (self.num_pages, self.page_size, self.num_heads, self.head_dim)
        eb = self.elem_bytes
        pool = torch.empty(shape, dtype=torch_dtype(self.dtype), device=device)
        pool.view(bits_dtype(eb)).fill_(_signed(SENTINEL_BITS[eb], eb))
        ref = torch.from_numpy(self.referenced_pages()).to(device)
        if len(ref):
            vals = self._values((len(ref),) + shape[1:], device, self._generator(device, 1))
            pool[ref] = vals
        return pool

    def make_src(self, device="cpu"):
        """[T, H, D] rows to scatter (new tokens in logical order)."""
        shape = (self.total_tokens, self.num_heads, self.head_dim)
        return self._values(shape, device, self._generator(device, 2))

    def make_scales(self, device="cpu"):
        """num_pages * page_size fp32 scales, uniform in [1e-3, 1e-1)."""
        import torch
        n = self.num_pages * self.page_size
        x = torch.rand(n, generator=self._generator(device, 3), device=device,
                       dtype=torch.float32)
        return x * (1e-1 - 1e-3) + 1e-3

    def describe(self):
        return {"workload": self.name, "dtype": self.dtype, "num_seqs": self.num_seqs,
                "total_tokens": self.total_tokens, "page_size": self.page_size,
                "num_heads": self.num_heads, "head_dim": self.head_dim,
                "num_pages": self.num_pages,
                "block_table_entries": self.num_block_entries,
                "index_type": np.dtype(self.index_dtype).name, **self.notes}


def _signed(bits, nbytes):
    """Bit pattern as the signed integer torch's fill_ expects for int types."""
    if nbytes == 1:
        return bits  # uint8
    top = 1 << (8 * nbytes - 1)
    return bits - (1 << (8 * nbytes)) if bits >= top else bits


def _pages_for(lengths, page_size):
    """Pages a sequence of each length occupies (ceil(length / page_size))."""
    return (np.asarray(lengths, dtype=np.int64) + page_size - 1) // page_size


def _ptr_from_counts(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])


# ---- the five workloads --------------------------------------------------

def tiny():
    """3 sequences of 40, 24 and 50 tokens, page_size 16, 20 pages; the block
    table is the first 10 entries of a seeded permutation of 0..19 and the
    first sequence holds one spare page beyond the 3 it needs; 4 heads x 8
    fp16 values uniform in [-1, 1]."""
    lens = np.array([40, 24, 50], dtype=np.uint32)
    bt = np.random.default_rng(0).permutation(20)[:10].astype(np.uint32)
    seq_ptr = np.array([0, 4, 6, 10], dtype=np.uint32)
    return Workload("tiny", "f16", 16, 4, 8, 20, np.uint32, bt, seq_ptr, lens,
                    values="uniform1", seed=0)


def decode():
    """64 sequences, lengths uniform in 1..2048, page_size 16, 32 heads x 128
    fp16 N(0,1), 12,000-page pool, unique random pages in a uint32 table."""
    rng = np.random.default_rng(1)
    lens = rng.integers(1, 2049, size=64).astype(np.uint32)
    n = _pages_for(lens, 16)
    bt = rng.permutation(12000)[: int(n.sum())].astype(np.uint32)
    return Workload("decode", "f16", 16, 32, 128, 12000, np.uint32, bt,
                    _ptr_from_counts(n).astype(np.uint32), lens, seed=1)


def prefix():
    """256 sequences sharing a 1024-token prefix (64 aliased pages), each
    followed by a private suffix of 16..512 tokens on fresh pages; page_size
    16, 8 heads x 128 bf16 N(0,1), 40,000-page pool, uint32 table."""
    rng = np.random.default_rng(2)
    suffix = rng.integers(16, 513, size=256)
    perm = rng.permutation(40000)
    shared = perm[:64]
    nxt = 64
    slices, lens = [], []
    for sl in suffix:
        own = int(_pages_for([sl], 16)[0])
        slices.append(np.concatenate([shared, perm[nxt: nxt + own]]))
        nxt += own
        lens.append(1024 + int(sl))
    bt = np.concatenate(slices).astype(np.uint32)
    seq_ptr = _ptr_from_counts([len(x) for x in slices]).astype(np.uint32)
    return Workload("prefix", "bf16", 16, 8, 128, 40000, np.uint32, bt, seq_ptr,
                    np.array(lens, dtype=np.uint32), seed=2,
                    notes={"shared_prefix_pages": 64})


def append():
    """512 decode sequences with a prior length L0 in 1..2047 (L0 mod 16 != 0),
    each writing 1 new token at position L0 into its partial trailing page,
    plus one 8,192-token prefill chunk written from position 0 into 512 fresh
    pages; page_size 16, 8 heads x 128 bf16 N(0,1), 60,000-page pool; the
    unused trailing slots of each written page are zeroed."""
    rng = np.random.default_rng(3)
    allowed = np.array([v for v in range(1, 2048) if v % 16 != 0])
    prior = rng.choice(allowed, size=512)
    perm = rng.permutation(60000)
    n_dec = _pages_for(prior, 16)
    counts = list(n_dec) + [512]
    bt = perm[: int(sum(counts))].astype(np.uint32)
    seq_ptr = _ptr_from_counts(counts).astype(np.uint32)
    lens = np.array([1] * 512 + [8192], dtype=np.uint32)
    start = np.array(list(prior) + [0], dtype=np.uint32)
    return Workload("append", "bf16", 16, 8, 128, 60000, np.uint32, bt, seq_ptr, lens,
                    seq_start=start, zero_tail=True, seed=3,
                    notes={"decode_seqs": 512, "prefill_tokens": 8192})


def quant():
    """1,024 sequences with log-normal lengths (median 1,024, sigma 1) capped to
    1..8,192; int8 pool of 200,000 pages x 16 slots x 8 heads x 128, values
    uniform in [-127, 127]; one fp32 scale per slot in [1e-3, 1e-1] (3.2M);
    unique random pages in a uint64 table; dequantised to bf16."""
    rng = np.random.default_rng(4)
    raw = np.exp(rng.normal(np.log(1024.0), 1.0, size=1024))
    lens = np.clip(np.rint(raw), 1, 8192).astype(np.uint64)
    n = _pages_for(lens, 16)
    bt = rng.permutation(200000)[: int(n.sum())].astype(np.uint64)
    return Workload("quant", "i8", 16, 8, 128, 200000, np.uint64, bt,
                    _ptr_from_counts(n).astype(np.uint64), lens, values="int8",
                    with_scales=True, seed=4)


CONFIGS = {"tiny": tiny, "decode": decode, "prefix": prefix, "append": append,
           "quant": quant}


def by_name(name):
    return CONFIGS[name]()


# ---- small random descriptors for fuzzing ---------------------------------

def random_small(seed, *, max_seqs=5, max_len=40, page_sizes=(1, 2, 3, 4, 5, 8, 16),
                 heads=(1, 2, 3), dims=(1, 2, 4, 8), dtypes=("f16", "bf16", "f32", "i8",
                                                            "u8", "f64"),
                 alias=True, spare_pages=True, index_dtype=None, with_start=False,
                 num_seqs=None):
    """A small, valid descriptor: random lengths (zero allowed), page size,
    heads, dims and dtype; optional aliasing of pages between sequences,
    optional spare pages at the end of a slice and optional start offsets.
    num_seqs fixes the sequence count (else it is drawn in 0..max_seqs)."""
    rng = np.random.default_rng(seed)
    P = int(rng.choice(page_sizes))
    H = int(rng.choice(heads))
    D = int(rng.choice(dims))
    dtype = str(rng.choice(list(dtypes)))
    S = int(rng.integers(0, max_seqs + 1)) if num_seqs is None else int(num_seqs)
    lens = rng.integers(0, max_len + 1, size=S)
    start = rng.integers(0, 2 * P + 1, size=S) if with_start else np.zeros(S, np.int64)
    need = _pages_for(lens + start, P)
    extra = rng.integers(0, 2, size=S) if spare_pages else np.zeros(S, np.int64)
    counts = need + extra
    K = int(counts.sum())
    N = max(1, K + int(rng.integers(0, 4)))
    bt = rng.permutation(N)[:K] if K else np.zeros(0, np.int64)
    if alias and K > 1:
        # let some entries name an earlier entry's page (aliasing)
        for k in range(1, K):
            if rng.random() < 0.3:
                bt[k] = bt[rng.integers(0, k)]
    idt = index_dtype or (np.uint32 if rng.random() < 0.5 else np.uint64)
    values = "int8" if dtype == "i8" else "normal"
    return Workload(f"random{seed}", dtype, P, H, D, N, idt, bt.astype(idt),
                    _ptr_from_counts(counts).astype(idt), lens.astype(idt),
                    seq_start=start.astype(idt) if with_start else None,
                    values=values, seed=seed)
