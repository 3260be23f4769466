"""GPU test of hp_gather_static, the gather whose workspace is the library's
own device array: through the C ABI, against hp_gather on the same
descriptor (bit for bit) and the oracle, on two calls in a row, the second
with a smaller input, for each path that uses the array: the plan arrays
above 4,096 sequences, the plan by choice from 512 sequences, and the
validator's words of a checked call."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_util import OnDevice, assert_bits_equal, host_bits, oracle_gather, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def hp():
    import block_table_gather_amd
    return block_table_gather_amd


def _case(seed, num_seqs):
    return workloads.random_small(seed, max_seqs=num_seqs, max_len=48, page_sizes=(4, 16),
                                  heads=(2,), dims=(64,), dtypes=("f16", "i8"),
                                  num_seqs=num_seqs)


def _run(hp, w, flags):
    d = OnDevice(w)
    T = w.total_tokens
    L = hp.lib()
    s = torch.cuda.current_stream().cuda_stream
    got = d.empty_out()
    assert L.hp_gather_static(d.desc.with_tokens(T), got.data_ptr(), flags, s) == 0
    ref = d.empty_out()
    ws = torch.empty(max(hp.workspace_bytes(d.desc, T), 256), dtype=torch.uint8, device=DEV)
    assert L.hp_gather(d.desc.with_tokens(T), ref.data_ptr(), ws.data_ptr(), ws.numel(),
                       flags, s) == 0
    torch.cuda.synchronize()
    g, r = host_bits(got), host_bits(ref)
    assert_bits_equal(g, r, "static vs workspace gather")
    assert_bits_equal(g, oracle_gather(d), "static gather vs oracle")


@pytest.mark.parametrize("flags", [0, 1, 4])  # plain, HP_FLAG_CHECKED, HP_FLAG_STREAM
def test_gather_static_two_calls(hp, flags):
    """Two calls in a row on the shared array, the second smaller: 6,000 then
    4,500 sequences (plan arrays required), 2,000 then 700 (plan by choice),
    then 64 (fused, the array untouched unless checked)."""
    for seed, n in ((900, 6000), (901, 4500), (902, 2000), (903, 700), (904, 64)):
        w = _case(seed, n)
        if flags == 4:  # the streaming hint asks for pages read once
            w = workloads.random_small(seed, max_seqs=n, max_len=48, page_sizes=(4, 16),
                                       heads=(2,), dims=(64,), dtypes=("f16", "i8"),
                                       num_seqs=n, alias=False)
        say("gather_static", flags, w.describe())
        _run(hp, w, flags)


def test_gather_static_checked_rejects(hp):
    """A checked call on a corrupted table reports the violation and writes
    nothing, with the verdict taken through the static array."""
    w = _case(905, 3000)
    bt = w.block_table.copy()
    bt[len(bt) // 3] = w.num_pages
    w.block_table = bt
    d = OnDevice(w)
    out = d.empty_out()
    with pytest.raises(hp.HpError, match="HP_ERR_PAGE_RANGE"):
        hp.gather_static(d.desc, out, checked=True)
    torch.cuda.synchronize()
    sentinel = workloads.SENTINEL_BITS[out.element_size()]
    assert np.all(host_bits(out) == sentinel)
