"""Pins of the CPU oracle to what the pages fix (no GPU).

Each test checks the oracle against a value the pages print, a closed form,
a special case that reduces to a library routine, or brute force; none of
them retypes the oracle's own formula.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from conftest import golden


# ---- address translation ---------------------------------------------------

def test_rust20_worked_example_scalar_indices():
    """[Rust20] worked example: T=(2,0,3,1), P=3, H_kv=2, d=2, one lane;
    lane 0, head 0, feature 0 of positions 0..6 sit at 24,26,28,0,2,4,36 in
    the [N,B,H_kv,P,d] array."""
    g = golden("rust20_worked_example.json")
    P, B, H, d = g["page_size"], g["batch"], g["kv_heads"], g["width"]
    strides = (B * H * P * d, d, P * d, 1)  # page, slot, head, feature of [N,B,H,P,d]
    bt = g["page_table"]
    seq_ptr = [0, len(bt)]
    got = [oracle.element_index(bt, seq_ptr, 0, p, g["head"], g["feature"], P, strides)
           for p in g["positions"]]
    assert got == g["expected_scalar_index"]
    # [Rust20] Include the batch, shared head and feature: a page spans
    # 1*2*3*2 = 12 scalars in each array, so page 2 starts at scalar 24
    assert strides[0] == g["page_slots"]
    assert oracle.element_index(bt, seq_ptr, 0, 0, 0, 0, P, strides) == g["page2_start"]
    # consecutive token rows of head 0 are 2 scalars apart (the feature width)
    assert (oracle.element_index(bt, seq_ptr, 0, 1, 0, 0, P, strides)
            - oracle.element_index(bt, seq_ptr, 0, 0, 0, 0, P, strides)) == g["row_step_head0"]
    # head 1's rows start 3*2 = 6 scalars after head 0's within the page
    assert (oracle.element_index(bt, seq_ptr, 0, 0, 1, 0, P, strides)
            - g["page2_start"]) == g["head1_offset_in_page"]
    # positions 9..11 are the reserved, unfilled rows of physical page 1
    for p in g["reserved_unfilled_positions"]:
        idx = oracle.element_index(bt, seq_ptr, 0, p, 0, 0, P, strides)
        assert idx // strides[0] == g["reserved_unfilled_physical_page"]


def test_rust20_example_under_interchange_layout():
    """The same table under the interchange layout [N,P,H,D]: the positions
    at page offset 0 keep their page start (page*P*H*D), the others step by a
    whole row (H*D = 4 scalars) instead of d = 2 -- the layouts differ only
    inside a page. Pinned to brute-force enumeration of the flat pool."""
    g = golden("rust20_worked_example.json")
    P, H, d, N = g["page_size"], g["kv_heads"], g["width"], 4
    bt = g["page_table"]
    # brute force: label every element of the [N,P,H,d] pool by its flat
    # position and read the label back through the slot list
    pool4 = [[[[((n * P + r) * H + h) * d + f for f in range(d)] for h in range(H)]
              for r in range(P)] for n in range(N)]
    rows = brute.gather(pool4, bt, [0, 4], [7])
    expected = [rows[p][0][0] for p in range(7)]
    strides = (P * H * d, H * d, d, 1)
    got = [oracle.element_index(bt, [0, 4], 0, p, 0, 0, P, strides) for p in range(7)]
    assert got == expected
    offset0 = [p for p in range(7) if p % P == 0]
    tut = g["expected_scalar_index"]
    assert all(got[p] == tut[p] for p in offset0)
    assert any(got[p] != tut[p] for p in range(7) if p % P)


def test_day51_block_lookup():
    """[Day51] token 42 with 16-token blocks reads block_table[42 // 16] = entry 2
    at offset 10 inside that block."""
    g = golden("day51_block.json")
    bt = [100, 200, 300, 400]
    P = g["block_size"]
    # strides (P, 1, 0, 0): the flat index is phys*P + offset
    idx = oracle.element_index(bt, [0, 4], 0, g["lookup_token"], 0, 0, P, (P, 1, 0, 0))
    assert idx == bt[g["lookup_block_index"]] * P + g["lookup_offset"]


# ---- gather on the spec's example ------------------------------------------

def _labelled_pool(N, P, H, D, dtype=np.uint16):
    """Pool whose every element holds its own flat position (distinct bits)."""
    return np.arange(N * P * H * D, dtype=np.int64).astype(dtype).reshape(N, P, H, D)


def test_hurray_example_gather():
    """[Hurray] Example: seq_ptr [0,2,3], block_table [0,1,0], P=4, N=5, H=2,
    D=8; sequences of 6 and 3 tokens; sequence 1 aliases page 0."""
    g = golden("hurray_example.json")
    N, P, H, D = g["num_pages"], g["page_size"], g["num_heads"], g["head_dim"]
    pool = _labelled_pool(N, P, H, D)
    assert pool.size == g["pool_values"]
    out = oracle.gather(pool, page_size=P, num_heads=H, head_dim=D,
                        block_table=g["block_table"], seq_ptr=g["seq_ptr"],
                        seq_lens=g["seq_lens"])
    assert out.shape == (g["total_tokens"], H, D)
    for row, (page, slot) in enumerate(g["row_sources"]):
        assert np.array_equal(out[row], pool[page, slot]), row
    # the aliased prefix reads back bit-identically
    assert np.array_equal(out[6:9].view(np.uint16), out[0:3].view(np.uint16))
    v = oracle.validate(rank=3, paged_axis=0, num_pages=N, page_size=P,
                        block_table=g["block_table"], seq_ptr=g["seq_ptr"],
                        seq_lens=g["seq_lens"], total_tokens=g["total_tokens"])
    assert v == ("valid", 0)


def test_hurray_example_never_reads_undefined_slots():
    """[Hurray] Partial trailing page: slots 2-3 of page 1 and slot 3 of page 0
    (for sequence 1) are undefined and must not be read."""
    g = golden("hurray_example.json")
    N, P, H, D = g["num_pages"], g["page_size"], g["num_heads"], g["head_dim"]
    pool = _labelled_pool(N, P, H, D)
    _, mark = oracle.gather(pool, page_size=P, num_heads=H, head_dim=D,
                            block_table=g["block_table"], seq_ptr=g["seq_ptr"],
                            seq_lens=g["seq_lens"], mark_reads=True)
    read = {(i // P, i % P) for i in np.flatnonzero(mark)}
    assert read == {tuple(x) for x in g["row_sources"]}
    for page, slot in g["undefined_slots"]:
        assert mark[page * P + slot] == 0


def test_prefix_sharing_slices():
    """[Hurray] Prefix Sharing: slices [12,5,7,9] and [12,5,7,3] share pages
    12, 5, 7; gathered rows of those pages are bit-identical across the two
    sequences, rows of pages 9 and 3 are not."""
    g = golden("hurray_prefix_sharing.json")
    P, H, D, N = 2, 2, 4, 16
    slices = g["slices"]
    bt = slices[0] + slices[1]
    seq_ptr = [0, 4, 8]
    lens = [4 * P, 4 * P]
    pool = _labelled_pool(N, P, H, D)
    out = oracle.gather(pool, page_size=P, num_heads=H, head_dim=D, block_table=bt,
                        seq_ptr=seq_ptr, seq_lens=lens)
    a, b = out[: 4 * P], out[4 * P:]
    shared = len(g["shared_pages"]) * P
    assert np.array_equal(a[:shared], b[:shared])
    assert not np.array_equal(a[shared:], b[shared:])
    assert np.array_equal(a[shared:], pool[g["private_pages"][0]])
    assert np.array_equal(b[shared:], pool[g["private_pages"][1]])
    v = oracle.validate(rank=3, paged_axis=0, num_pages=N, page_size=P, block_table=bt,
                        seq_ptr=seq_ptr, seq_lens=lens, total_tokens=8 * P)
    assert v == ("valid", 0), "aliasing is expressible and not rejected"


def test_empty_batch():
    """[Hurray] Buffer Table note: num_seqs = 0, seq_ptr = [0], empty table."""
    v = oracle.validate(rank=3, paged_axis=0, num_pages=0, page_size=16,
                        block_table=[], seq_ptr=[0], seq_lens=[], total_tokens=0)
    assert v == ("valid", 0)
    pool = np.zeros((1, 16, 2, 4), np.uint16)
    out = oracle.gather(pool, page_size=16, num_heads=2, head_dim=4, block_table=[],
                        seq_ptr=[0], seq_lens=[])
    assert out.shape == (0, 2, 4)
    res = oracle.scatter(pool, np.zeros((0, 2, 4), np.uint16), page_size=16, num_heads=2,
                         head_dim=4, block_table=[], seq_ptr=[0], seq_lens=[],
                         zero_tail=True)
    assert np.array_equal(res, pool)


# ---- validator ---------------------------------------------------------------

BASE = dict(rank=3, paged_axis=0, num_pages=8, page_size=4,
            block_table=[0, 1, 2, 3, 4], seq_ptr=[0, 2, 2, 5], seq_lens=[7, 0, 9],
            total_tokens=16)


def _with(**kw):
    d = dict(BASE)
    d.update(kw)
    return d


@pytest.mark.parametrize("case,expected", [
    ({}, ("valid", 0)),
    (dict(rank=2), ("rank", 0)),                                   # Description
    (dict(rank=4), ("rank", 0)),
    (dict(paged_axis=1), ("paged_axis", 0)),                       # invariant (6)
    (dict(seq_ptr=[1, 2, 2, 5]), ("seq_ptr_first", 0)),            # invariant (1)
    (dict(seq_ptr=[0, 2, 2, 4]), ("seq_ptr_last", 3)),             # invariant (1)
    (dict(seq_ptr=[0, 3, 2, 5]), ("seq_ptr_order", 1)),            # invariant (2)
    (dict(block_table=[0, 1, 8, 3, 9]), ("page_range", 2)),        # invariant (3)
    (dict(seq_lens=[9, 0, 9], total_tokens=18), ("seq_len", 0)),   # partial page rule
    (dict(seq_lens=[8, 1, 9], total_tokens=18), ("seq_len", 1)),
    (dict(total_tokens=15), ("total_tokens", 0)),                  # Logical Shape
    (dict(seq_ptr=[1, 3, 2, 4], block_table=[0, 1, 9, 3]), ("seq_ptr_first", 0)),
    (dict(block_table=[0, 1, 2, 3, 4, 5]), ("seq_ptr_last", 3)),
])
def test_validator_cases(case, expected):
    args = _with(**case)
    assert oracle.validate(**args) == expected
    fails = brute.validate(args["rank"], args["paged_axis"], args["num_pages"],
                           args["page_size"], args["block_table"], args["seq_ptr"],
                           args["seq_lens"], args["total_tokens"])
    assert (fails[0] if fails else ("valid", 0)) == expected


def test_validator_scatter_window():
    """With start offsets the last written position must still lie in the
    slice: start 6 + 3 tokens = 9 > 2 pages * 4 slots."""
    args = _with(seq_lens=[3, 0, 9], total_tokens=12)
    assert oracle.validate(**args, seq_start=[5, 0, 0]) == ("valid", 0)
    assert oracle.validate(**args, seq_start=[6, 0, 0]) == ("seq_len", 0)


# ---- disjoint writes (a scatter's destinations) ------------------------------

def _dw(P, bt, sp, lens, starts=None, zero_tail=False, N=None):
    """Oracle and brute force together (they must agree)."""
    N = (max(bt) + 1) if N is None else N
    got = oracle.disjoint_writes(num_pages=N, page_size=P, block_table=bt, seq_ptr=sp,
                                 seq_lens=lens, seq_start=starts, zero_tail=zero_tail)
    assert got == brute.disjoint_writes(P, bt, sp, lens, starts, zero_tail)
    return got


def test_disjoint_writes_hurray_example():
    """[Hurray] Example read as a scatter: sequence 1's slice names page 0,
    which sequence 0 fills too, so both write slots 0-2 of page 0: sequence 0
    is the first whose writes repeat. Writing only page 1 (sequence 0's
    tokens 4-5) and page 0 (sequence 1) is disjoint."""
    g = golden("hurray_example.json")
    P, bt, sp, lens = g["page_size"], g["block_table"], g["seq_ptr"], g["seq_lens"]
    assert _dw(P, bt, sp, lens, N=g["num_pages"]) == 0
    assert _dw(P, bt, sp, [2, 3], starts=[4, 0], N=g["num_pages"]) is None
    # with the tails zeroed, page 1's slots 2-3 are sequence 0's alone, but
    # sequence 1's tail (slot 3 of page 0) is sequence 0's token 3 only when
    # sequence 0 writes page 0
    assert _dw(P, bt, sp, [2, 3], starts=[4, 0], zero_tail=True, N=g["num_pages"]) is None
    assert _dw(P, bt, sp, [6, 3], zero_tail=True, N=g["num_pages"]) == 0


def test_disjoint_writes_prefix_sharing_slices():
    """[Hurray] Prefix Sharing slices [12,5,7,9] and [12,5,7,3]: writing both
    sequences' full slices writes pages 12, 5 and 7 twice; appending to the
    private last pages only (start 3 P) is disjoint."""
    g = golden("hurray_prefix_sharing.json")
    P = 2
    bt = g["slices"][0] + g["slices"][1]
    sp = [0, 4, 8]
    assert _dw(P, bt, sp, [4 * P, 4 * P], N=16) == 0
    assert _dw(P, bt, sp, [P, P], starts=[3 * P, 3 * P], N=16) is None
    assert _dw(P, bt, sp, [1, 1], starts=[3 * P, 3 * P], zero_tail=True, N=16) is None


def test_disjoint_writes_through_the_tail_only():
    """Two windows of one page: tokens 0-1 (sequence 0) and 2-3 (sequence 1)
    are disjoint, but zeroing sequence 0's tail writes slots 2-3 again."""
    bt, sp = [5, 5], [0, 1, 2]
    assert _dw(4, bt, sp, [2, 2], starts=[0, 2]) is None
    assert _dw(4, bt, sp, [2, 2], starts=[0, 2], zero_tail=True) == 0
    # swapped windows: sequence 0's last token ends the page (no tail), and
    # sequence 1's tail rewrites sequence 0's slots, so 0 is still the first
    # sequence with a repeated slot
    assert _dw(4, bt, sp, [2, 2], starts=[2, 0]) is None
    assert _dw(4, bt, sp, [2, 2], starts=[2, 0], zero_tail=True) == 0


def test_disjoint_writes_page_repeated_in_one_slice():
    """A slice that names page 3 twice writes its slots twice by itself."""
    assert _dw(4, [1, 3, 3], [0, 1, 3], [4, 8]) == 1
    assert _dw(4, [1, 3, 3], [0, 1, 3], [4, 4]) is None  # only the first page written


def test_disjoint_writes_reports_the_smallest_sequence():
    """Sequences 2 and 5 share page 7; the others are disjoint: 2."""
    bt = [0, 1, 7, 3, 4, 7]
    sp = list(range(7))
    assert _dw(4, bt, sp, [4] * 6) == 2
    assert _dw(4, bt, sp, [4, 4, 4, 4, 4, 0]) is None


def test_disjoint_writes_brute_force():
    """Random tiny scatters with aliased slices, start offsets and both tail
    modes: the oracle agrees with the brute force (_dw asserts it)."""
    rng = np.random.default_rng(77)
    found = clean = 0
    for _ in range(400):
        P = int(rng.integers(1, 5))
        N = int(rng.integers(1, 7))
        S = int(rng.integers(1, 6))
        counts = rng.integers(0, 4, size=S)
        bt = [int(x) for x in rng.integers(0, N, size=int(counts.sum()))]
        sp = [0] + [int(x) for x in np.cumsum(counts)]
        lens, starts = [], []
        for c in counts:
            L = int(rng.integers(0, c * P + 1))
            lens.append(L)
            starts.append(int(rng.integers(0, c * P - L + 1)))
        for zt in (False, True):
            r = _dw(P, bt, sp, lens, starts, zt, N=N)
            found += r is not None
            clean += r is None
    assert found > 100 and clean > 100


# ---- byte accounting ---------------------------------------------------------

def test_rust20_payload():
    g = golden("rust20_payload.json")
    m = g["main"]
    p = oracle.payload(capacity=m["capacity"], page_tokens=m["page_tokens"],
                       length=m["length"], batch=m["batch"], kv_heads=m["kv_heads"],
                       width=m["width"], elem_bytes=g["elem_bytes"])
    for key in ("reserved_pages", "active_pages", "allocated_slots", "live_slots",
                "unused_slots", "tail_slots", "inactive_slots", "allocated_bytes",
                "live_bytes", "unused_bytes", "tail_bytes", "inactive_bytes"):
        assert p[key] == m[key], key
    assert m["layers"] * p["allocated_bytes"] == m["all_layers_allocated_bytes"]


def test_rust20_rounded_reservation():
    g = golden("rust20_payload.json")
    r = g["rounded"]
    p = oracle.payload(capacity=r["capacity"], page_tokens=r["page_tokens"],
                       length=r["length"], batch=r["batch"], kv_heads=r["kv_heads"],
                       width=r["width"], elem_bytes=g["elem_bytes"])
    assert p["reserved_pages"] == r["reserved_pages"]
    assert p["allocated_slots"] == r["paged_slots"]
    assert p["contiguous_slots"] == r["contiguous_slots"]
    extra = p["allocated_slots"] - p["contiguous_slots"]
    assert extra == r["extra_slots"] and extra * g["elem_bytes"] == r["extra_bytes"]
    assert p["live_slots"] == 0 and p["unused_slots"] == p["allocated_slots"]
    q = oracle.payload(capacity=r["same_at_capacity"], page_tokens=r["page_tokens"],
                       length=0, batch=1, kv_heads=2, width=2, elem_bytes=8)
    assert q["allocated_slots"] == q["contiguous_slots"] == r["slots_at_capacity_12"]


def test_day51_block_bytes():
    """[Day51] 2 (K,V) x 16 x 32 x 128 x 2 bytes = 262,144 bytes per block and
    layer; x32 layers = 8 MiB."""
    g = golden("day51_block.json")
    p = oracle.payload(capacity=g["block_size"], page_tokens=g["block_size"],
                       length=g["block_size"], batch=1, kv_heads=g["num_heads"],
                       width=g["head_dim"], elem_bytes=g["dtype_bytes"])
    assert p["allocated_bytes"] == g["bytes_per_kv_block_per_layer"]
    assert p["live_bytes"] == p["allocated_bytes"] and p["tail_bytes"] == 0
    assert p["allocated_bytes"] * g["layers"] == g["bytes_per_block_all_layers"]


def test_day51_trace_blocks():
    """[Day51] trace: prompts of 40, 24, 50 tokens need 3, 2, 4 blocks; the
    payload's active page count is that ceiling."""
    g = golden("day51_block.json")
    for n, need in zip(g["trace_prompt_lengths"], g["trace_blocks_needed"]):
        p = oracle.payload(capacity=64, page_tokens=g["block_size"], length=n, batch=1,
                           kv_heads=1, width=1, elem_bytes=1)
        assert p["active_pages"] == need


# ---- rounding ----------------------------------------------------------------

def _torch_bf16_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_library_rounding():
    """fp32 -> bf16 round-to-nearest-even equals torch's CPU conversion on every
    high half with the discarded half at its edge cases (0, 1, just below /
    at / above the halfway point, all ones) and on random patterns."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    rng = np.random.default_rng(7)
    bits = np.concatenate([(hi[:, None] | lows[None, :]).ravel(),
                           rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)])
    x = bits.view(np.float32)
    got = oracle.bf16_rne(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN with its sign
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all((g & 0x7F) != 0)
    assert np.array_equal(g >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_bf16_rne_ties_to_even():
    """Closed forms: exactly representable values are unchanged; halfway
    values go to the even neighbour; overflow past the largest finite value
    gives infinity."""
    ones = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F808001, 0x7F7FFFFF,
                     0x7F7F8000, 0x00008000, 0x00018000], dtype=np.uint32)
    expect = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x7F80, 0x7F80, 0x0000, 0x0002],
                      dtype=np.uint16)
    assert np.array_equal(oracle.bf16_rne(ones.view(np.float32)), expect)


def test_dequant_matches_library_arithmetic():
    """Every int8 value times a dense sweep of fp32 scales, dequantised through
    a one-page table: equals torch's CPU (q.float() * s).to(bfloat16) bit for
    bit (a single IEEE binary32 multiply, then round to nearest even)."""
    P, H, D = 4, 1, 256
    rng = np.random.default_rng(11)
    scales = np.concatenate([np.geomspace(1e-3, 1e-1, 2048, dtype=np.float32),
                             rng.uniform(1e-3, 1e-1, 2048).astype(np.float32),
                             np.array([1.0, 0.5, 3.0, 1e-30, 2.5e-39, 1e30, -0.25,
                                       np.float32(1 / 3)], dtype=np.float32)])
    q = np.arange(-128, 128, dtype=np.int8)
    n_pages = -(-len(scales) // P)
    sc = np.zeros(n_pages * P, np.float32)
    sc[: len(scales)] = scales
    pool = np.broadcast_to(q, (n_pages, P, H, D)).copy()
    bt = np.arange(n_pages)
    got = oracle.gather_dequant(pool, sc, page_size=P, num_heads=H, head_dim=D,
                                block_table=bt, seq_ptr=[0, n_pages],
                                seq_lens=[n_pages * P])
    ref = (torch.from_numpy(pool.reshape(n_pages * P, H * D)).float()
           * torch.from_numpy(sc)[:, None]).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16).reshape(got.shape)
    assert np.array_equal(got, ref)


def test_day51_copy_on_write_keeps_the_other_request_intact():
    """[Day51] Copy-on-write: requests D and E share a 24-token system prompt
    (blocks 0 and 1; block 1 half full) and each has a private block. Before
    E writes its next token into the shared half-full block, that block is
    copied to a fresh one and E's table points there ([Hurray] Prefix
    Sharing: aliasing is static structure; the copy is the writer's job).
    D's gathered rows are unchanged, E's prefix rows equal D's, E's new token
    is in place, and the shared page itself is untouched."""
    P, H, D, N = 16, 2, 4, 8
    pool = _labelled_pool(N, P, H, D)
    shared = [0, 1]
    bt_d, bt_e = shared + [2], shared + [3]
    sp = [0, 3, 6]
    lens = [24, 24]                                  # both hold only the prompt
    kw = dict(page_size=P, num_heads=H, head_dim=D)
    before = oracle.gather(pool, block_table=bt_d + bt_e, seq_ptr=sp, seq_lens=lens, **kw)
    # copy-on-write: block 1 -> fresh block 4 for E, then E appends at position 24
    pool2, _ = oracle.copy_pages(pool, [1], [4], **kw)
    bt_e2 = [0, 4, 3]
    new_row = np.full((1, H, D), 0x7777, dtype=pool.dtype)
    pool3 = oracle.scatter(pool2, new_row, block_table=bt_e2, seq_ptr=[0, 3], seq_lens=[1],
                           seq_start=[24], **kw)
    after = oracle.gather(pool3, block_table=bt_d + bt_e2, seq_ptr=sp, seq_lens=[24, 25], **kw)
    assert np.array_equal(after[:24], before[:24])           # D unchanged
    assert np.array_equal(after[24:48], before[:24])         # E's prefix == D's
    assert np.all(after[48] == 0x7777)                       # E's new token
    assert np.array_equal(pool3[1], pool[1])                 # the shared page untouched
    assert np.array_equal(pool3[4, 8], new_row[0])           # slot 24 mod 16 of the copy


@pytest.mark.parametrize("scheme,axis,block,accept", [
    ("per_tensor", 0, 0, True),          # composes normally
    ("per_channel", 1, 0, True),         # num_heads axis
    ("per_channel", 2, 0, True),         # head_dim axis
    ("per_channel", 0, 0, False),        # paged axis: forbidden
    ("per_block_affine", 0, 16, True),   # axis 0, block_size == page_size
    ("per_block_affine", 0, 8, False),   # block_size != page_size: must reject
    ("per_block_affine", 1, 16, False),  # axis != 0: must reject
    ("per_block_affine", 2, 16, False),
])
def test_hurray_scheme_composition_rules(scheme, axis, block, accept):
    """[Hurray] Per-scheme composition: which quantization schemes a reader
    accepts on a block-paged tensor with page_size 16."""
    assert oracle.quant_accepts(scheme, axis, block, 16) == accept
