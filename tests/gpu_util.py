"""Helpers for the GPU parity tests: device copies of a workload, host bit
views of device tensors, and the oracle's result for the same inputs."""
import sys

import numpy as np
import torch

import oracle
import workloads


def say(*msg):
    """Name the case before any GPU work (a dying box returns only the tail)."""
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def idx_tensor(a, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32).copy()).to(dev)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64).copy()).to(dev)
    raise TypeError(a.dtype)


def host_bits(t):
    eb = t.element_size()
    return (t.detach().contiguous().view(workloads.bits_dtype(eb)).cpu().numpy()
            .view(workloads.np_bits_dtype(eb)))


def fill_bits(t, bits):
    eb = t.element_size()
    t.view(workloads.bits_dtype(eb)).fill_(workloads._signed(bits, eb))
    return t


class OnDevice:
    """A workload's descriptor tensors (and pool, scales) on the GPU."""

    def __init__(self, w, dev="cuda", pool=None):
        import block_table_gather_amd as hp
        self.w = w
        self.dev = dev
        self.pool = w.make_pool(dev) if pool is None else pool
        self.bt = idx_tensor(w.block_table.astype(w.index_dtype), dev)
        self.sp = idx_tensor(w.seq_ptr.astype(w.index_dtype), dev)
        self.sl = idx_tensor(w.seq_lens.astype(w.index_dtype), dev)
        self.ss = (idx_tensor(w.seq_start.astype(w.index_dtype), dev)
                   if w.seq_start is not None else None)
        self.scales = w.make_scales(dev) if (w.with_scales or w.dtype == "i8") else None
        self.desc = hp.Descriptor(self.pool, self.bt, self.sp, self.sl, scales=self.scales)

    def oracle_kw(self, with_start=False):
        w = self.w
        kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
                  block_table=w.block_table, seq_ptr=w.seq_ptr, seq_lens=w.seq_lens)
        if with_start:
            kw["seq_start"] = w.seq_start
        return kw

    def empty_out(self, dtype=None, sentinel=True):
        w = self.w
        out = torch.empty((w.total_tokens, w.num_heads, w.head_dim),
                          dtype=dtype or self.pool.dtype, device=self.dev)
        if sentinel:
            fill_bits(out, workloads.SENTINEL_BITS[out.element_size()])
        return out


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got.ravel() != want.ravel())
        raise AssertionError(f"{what}: {len(bad)} of {got.size} elements differ; first at "
                             f"{bad[:8].tolist()}: got {got.ravel()[bad[:8]].tolist()} "
                             f"want {want.ravel()[bad[:8]].tolist()}")


def bf16_bits_equal(got, want, what=""):
    """bf16 bit patterns equal, except that any NaN matches any NaN."""
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    assert_bits_equal(np.where(nan_g, 0, got), np.where(nan_w, 0, want), what)


def oracle_gather(d):
    return oracle.gather(host_bits(d.pool), **d.oracle_kw())


def empty_seq_workload(dtype, seed):
    """Nine sequences, four of them empty (the first, the last and two between;
    two of the empty ones still name a page), ten kv heads of 128 with 16-token
    pages: three head groups on the matrix cores, the last holding two kv heads."""
    lens = np.array([0, 37, 0, 0, 130, 1, 0, 64, 0], np.uint32)
    npg = [1, 3, 0, 1, 9, 1, 0, 4, 0]
    sp = np.concatenate([[0], np.cumsum(npg)]).astype(np.uint32)
    rng = np.random.default_rng(seed)
    bt = rng.permutation(40)[: int(sp[-1])].astype(np.uint32)
    values = "int8" if dtype == "i8" else "normal"
    return workloads.Workload("empty-seqs", dtype, 16, 10, 128, 40, np.uint32, bt, sp, lens,
                              values=values, with_scales=dtype == "i8", seed=seed)

