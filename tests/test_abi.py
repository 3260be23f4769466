"""The C-ABI library loads, exports every symbol include/hp.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed: every
call here returns before the library touches the device)."""
import ctypes
import os
import re

import pytest

import block_table_gather_amd as hp
from conftest import ROOT

HDR = os.path.join(ROOT, "include", "hp.h")
L = hp.lib()
S = hp.CODE
ALIGNED = 0x7F0000000000  # a fake, 256-byte aligned device address (never dereferenced)


def declared_functions():
    text = open(HDR).read()
    return re.findall(r"^(?:hp_status|size_t|const char \*)\s*(hp_\w+)\(", text, re.M)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == {"hp_workspace_bytes", "hp_validate", "hp_gather", "hp_scatter",
                          "hp_gather_dequant", "hp_status_str", "hp_last_hip_error",
                          "hp_gather_batch", "hp_scatter_batch", "hp_gather_dequant_batch",
                          "hp_copy_pages", "hp_copy_pages_batch", "hp_gather_dequant_q",
                          "hp_paged_attention", "hp_paged_attention_q8", "hp_attention_plan",
                          "hp_attention_workspace_bytes",
                          "hp_scatter_quant", "hp_validate_async", "hp_validate_verdict",
                          "hp_gather_static", "hp_validate_writes",
                          "hp_disjoint_workspace_bytes"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code, name in hp.STATUS.items():
        assert hp.status_str(code).startswith(name)
    assert hp.status_str(999) == "unknown hp_status"
    assert hp.last_hip_error() == "hipSuccess"


def desc(**kw):
    d = hp.HpDesc()
    d.rank, d.paged_axis, d.index_type, d.dtype = 3, 0, hp.HP_INDEX_U32, hp.DTYPE["f16"]
    d.page_size, d.num_heads, d.head_dim = 16, 4, 8
    d.num_pages, d.num_seqs, d.num_block_entries, d.total_tokens = 20, 3, 10, 114
    d.page_pool = ALIGNED
    d.block_table = ALIGNED + 0x100000
    d.seq_ptr = ALIGNED + 0x200000
    d.seq_lens = ALIGNED + 0x300000
    d.scales = None
    for k, v in kw.items():
        setattr(d, k, v)
    return d


OUT = ALIGNED + 0x100000000


def gather(d, out=OUT, ws=None, n=0, flags=0):
    return L.hp_gather(ctypes.byref(d) if d is not None else None, out, ws, n, flags, None)


@pytest.mark.parametrize("fields,code", [
    (dict(rank=2), "HP_ERR_RANK"),
    (dict(rank=4), "HP_ERR_RANK"),
    (dict(paged_axis=1), "HP_ERR_PAGED_AXIS"),
    (dict(has_shard=1), "HP_ERR_SHARDED"),
    (dict(index_type=2), "HP_ERR_INDEX_TYPE"),
    (dict(dtype=0), "HP_ERR_DTYPE"),
    (dict(dtype=99), "HP_ERR_DTYPE"),
    (dict(byte_offset=64), "HP_ERR_ARG"),
    (dict(page_size=0), "HP_ERR_ARG"),
    (dict(num_heads=0), "HP_ERR_ARG"),
    (dict(head_dim=0), "HP_ERR_ARG"),
    (dict(num_pages=1 << 62), "HP_ERR_ARG"),                       # pool bytes overflow
    (dict(num_heads=1 << 20, head_dim=1 << 12), "HP_ERR_ARG"),     # row too large
    (dict(num_pages=(1 << 32) + 1), "HP_ERR_INDEX_TYPE"),          # uint32 too narrow
    (dict(seq_ptr=None), "HP_ERR_NULL"),
    (dict(block_table=None), "HP_ERR_NULL"),
    (dict(seq_lens=None), "HP_ERR_NULL"),
    (dict(page_pool=None), "HP_ERR_NULL"),
    (dict(page_pool=ALIGNED + 32), "HP_ERR_ALIGN"),                # descriptor buffers: 64 B
    (dict(block_table=ALIGNED + 4), "HP_ERR_ALIGN"),
    (dict(seq_ptr=ALIGNED + 8), "HP_ERR_ALIGN"),
    (dict(seq_lens=ALIGNED + 2), "HP_ERR_ALIGN"),
])
def test_descriptor_rejections(fields, code):
    d = desc(**fields)
    assert gather(d) == S[code]
    assert L.hp_scatter(ctypes.byref(d), OUT, None, None, 0, 0, None) == S[code]
    res = hp.HpValidateResult()
    assert L.hp_validate(ctypes.byref(d), None, OUT, 4096, ctypes.byref(res), None) == S[code]
    assert res.code == S[code]
    assert L.hp_workspace_bytes(ctypes.byref(d)) == 0


def test_null_descriptor():
    assert gather(None) == S["HP_ERR_NULL"]
    assert L.hp_scatter(None, OUT, None, None, 0, 0, None) == S["HP_ERR_NULL"]
    assert L.hp_gather_dequant(None, OUT, hp.DTYPE["bf16"], None, 0, 0, None) == S["HP_ERR_NULL"]
    assert L.hp_validate(None, None, None, 0, None, None) == S["HP_ERR_NULL"]
    assert L.hp_workspace_bytes(None) == 0


def test_call_buffer_rejections():
    d = desc()
    assert gather(d, out=None) == S["HP_ERR_NULL"]
    assert gather(d, out=OUT + 1) == S["HP_ERR_ALIGN"]
    assert gather(d, out=ALIGNED + 64) == S["HP_ERR_ARG"]            # overlaps the pool
    assert gather(d, flags=16) == S["HP_ERR_ARG"]                    # unknown flag
    assert L.hp_scatter(ctypes.byref(d), OUT, None, None, 0, hp.HP_FLAG_STREAM, None) == \
        S["HP_ERR_ARG"]                                              # gather-only hint
    assert gather(d, flags=hp.HP_FLAG_ZERO_TAIL) == S["HP_ERR_ARG"]  # scatter-only flag
    assert gather(d, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    assert gather(d, ws=OUT + 0x100000, n=255, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    assert gather(d, ws=OUT + 0x100004, n=4096, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_ALIGN"]
    sc = ctypes.byref(d)
    assert L.hp_scatter(sc, None, None, None, 0, 0, None) == S["HP_ERR_NULL"]
    assert L.hp_scatter(sc, OUT, ALIGNED + 0x400002, None, 0, 0, None) == S["HP_ERR_ALIGN"]
    assert L.hp_scatter(sc, OUT, None, None, 0, 16, None) == S["HP_ERR_ARG"]
    res = hp.HpValidateResult()
    assert L.hp_validate(sc, None, None, 0, ctypes.byref(res), None) == S["HP_ERR_WORKSPACE"]
    assert L.hp_validate(sc, None, OUT, 16, ctypes.byref(res), None) == S["HP_ERR_WORKSPACE"]


def test_dequant_rejections():
    q = desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500000)
    bf16 = hp.DTYPE["bf16"]
    call = lambda d, out=OUT, od=bf16: L.hp_gather_dequant(ctypes.byref(d), out, od, None, 0, 0, None)  # noqa: E731
    assert call(desc(scales=ALIGNED + 0x500000)) == S["HP_ERR_DTYPE"]   # f16 pool
    assert call(q, od=hp.DTYPE["f16"]) == S["HP_ERR_DTYPE"]
    assert call(desc(dtype=hp.DTYPE["i8"])) == S["HP_ERR_NULL"]        # no scales
    assert call(desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500004)) == S["HP_ERR_ALIGN"]
    assert call(q, out=None) == S["HP_ERR_NULL"]
    assert call(q, out=OUT + 1) == S["HP_ERR_ALIGN"]
    assert call(q, out=ALIGNED + 0x500000) == S["HP_ERR_ARG"]          # overlaps scales


def quant(scheme, axis=0, block_size=16, scales=ALIGNED + 0x500000, zero_points=None):
    return hp.HpQuant(hp.QUANT_SCHEME[scheme] if isinstance(scheme, str) else scheme, axis,
                      block_size, scales, zero_points)


def dq_q(d, q, out=OUT, od=None, flags=0):
    od = hp.DTYPE["bf16"] if od is None else od
    return L.hp_gather_dequant_q(ctypes.byref(d) if d is not None else None,
                                 ctypes.byref(q) if q is not None else None,
                                 out, od, None, 0, flags, None)


@pytest.mark.parametrize("scheme,axis,block,code", [
    ("per_tensor", 0, 16, "HP_OK"),
    ("per_tensor", 2, 7, "HP_OK"),                 # axis and block size are not used
    ("per_channel", 1, 16, "HP_OK"),
    ("per_channel", 2, 16, "HP_OK"),
    ("per_channel", 0, 16, "HP_ERR_QUANT"),        # channel along the paged axis
    ("per_channel", 3, 16, "HP_ERR_QUANT"),
    ("per_block_affine", 0, 16, "HP_OK"),
    ("per_block_affine", 0, 8, "HP_ERR_QUANT"),    # block must equal the page
    ("per_block_affine", 0, 32, "HP_ERR_QUANT"),
    ("per_block_affine", 1, 16, "HP_ERR_QUANT"),   # blocks not along the paged axis
    (0x04, 0, 16, "HP_ERR_QUANT"),                 # unknown scheme tag
    (0x00, 0, 16, "HP_ERR_QUANT"),
])
def test_quant_scheme_acceptance(scheme, axis, block, code):
    """The composition rules; an accepted scheme with total_tokens == 0 returns
    HP_OK before touching the device."""
    d = desc(dtype=hp.DTYPE["i8"], total_tokens=0)
    assert dq_q(d, quant(scheme, axis, block)) == S[code]
    assert dq_q(desc(dtype=hp.DTYPE["u8"], total_tokens=0), quant(scheme, axis, block)) == S[code]


def test_quant_rejections():
    q8 = desc(dtype=hp.DTYPE["i8"])
    pt = quant("per_tensor")
    assert dq_q(None, pt) == S["HP_ERR_NULL"]
    assert dq_q(q8, None) == S["HP_ERR_NULL"]
    assert dq_q(desc(), pt) == S["HP_ERR_DTYPE"]                       # f16 pool
    assert dq_q(q8, pt, od=hp.DTYPE["f32"]) == S["HP_ERR_DTYPE"]
    assert dq_q(q8, quant("per_tensor", scales=None)) == S["HP_ERR_NULL"]
    assert dq_q(q8, quant("per_tensor", scales=ALIGNED + 0x500004)) == S["HP_ERR_ALIGN"]
    assert dq_q(q8, quant("per_tensor", zero_points=ALIGNED + 0x600001)) == S["HP_ERR_ALIGN"]
    assert dq_q(q8, pt, out=None) == S["HP_ERR_NULL"]
    assert dq_q(q8, pt, out=OUT + 1) == S["HP_ERR_ALIGN"]
    assert dq_q(q8, pt, out=ALIGNED + 0x500000) == S["HP_ERR_ARG"]    # overlaps scales
    assert dq_q(q8, quant("per_tensor", zero_points=OUT + 128)) == S["HP_ERR_ARG"]
    assert dq_q(q8, pt, out=ALIGNED + 64) == S["HP_ERR_ARG"]          # overlaps the pool
    assert dq_q(q8, pt, flags=hp.HP_FLAG_STREAM) == S["HP_ERR_ARG"]
    assert dq_q(q8, pt, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    # the descriptor's own scales play no part
    assert dq_q(desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500004, total_tokens=0), pt) == \
        S["HP_OK"]


def attn(d, v=ALIGNED + 0x40000000, q=ALIGNED + 0x50000000, hq=8, out=OUT, od=None, ws=None,
         n=None, flags=0):
    od = hp.DTYPE["f32"] if od is None else od
    if ws is None:
        ws = ALIGNED + 0x200000000
        n = 1 << 30 if n is None else n
    return L.hp_paged_attention(ctypes.byref(d) if d is not None else None, v, q, hq, 0.125,
                                out, od, ws, n or 0, flags, None)


def test_attention_rejections():
    d = desc(num_seqs=0, num_block_entries=0, total_tokens=0)     # accepted shape, no work
    assert attn(d) == S["HP_OK"]
    assert attn(None) == S["HP_ERR_NULL"]
    f = desc()
    assert attn(desc(dtype=hp.DTYPE["f32"])) == S["HP_ERR_DTYPE"]
    assert attn(desc(dtype=hp.DTYPE["i8"])) == S["HP_ERR_DTYPE"]
    assert attn(f, od=hp.DTYPE["bf16"]) == S["HP_ERR_DTYPE"]
    assert attn(desc(head_dim=24)) == S["HP_ERR_ARG"]              # not a supported width
    assert attn(desc(head_dim=512)) == S["HP_ERR_ARG"]
    assert attn(f, hq=6) == S["HP_ERR_ARG"]                        # not a multiple of 4 kv heads
    assert attn(f, hq=0) == S["HP_ERR_ARG"]
    assert attn(desc(page_size=1 << 17)) == S["HP_ERR_ARG"]
    assert attn(f, flags=hp.HP_FLAG_ZERO_TAIL) == S["HP_ERR_ARG"]
    assert attn(f, v=None) == S["HP_ERR_NULL"]
    assert attn(f, q=None) == S["HP_ERR_NULL"]
    assert attn(f, out=None) == S["HP_ERR_NULL"]
    assert attn(f, v=ALIGNED + 0x40000020) == S["HP_ERR_ALIGN"]
    assert attn(f, q=ALIGNED + 0x50000008) == S["HP_ERR_ALIGN"]
    assert attn(f, out=OUT + 4) == S["HP_ERR_ALIGN"]
    assert attn(f, ws=None, n=0) == S["HP_ERR_WORKSPACE"]
    need = L.hp_attention_workspace_bytes(ctypes.byref(f), 8)
    assert need > 256
    assert attn(f, n=need - 1) == S["HP_ERR_WORKSPACE"]
    assert attn(f, ws=ALIGNED + 0x200000000 + 64, n=need) == S["HP_ERR_ALIGN"]
    assert attn(f, out=ALIGNED + 64) == S["HP_ERR_ARG"]            # out overlaps the K pool
    assert attn(f, out=ALIGNED + 0x40000000) == S["HP_ERR_ARG"]    # out overlaps the V pool
    assert attn(f, ws=ALIGNED + 0x50000000, n=need) == S["HP_ERR_ARG"]  # workspace over q
    assert attn(f, out=ALIGNED + 0x200000000) == S["HP_ERR_ARG"]   # out over the workspace


def test_attention_workspace_bytes():
    f = desc()
    assert L.hp_attention_workspace_bytes(None, 8) == 0
    assert L.hp_attention_workspace_bytes(ctypes.byref(desc(dtype=hp.DTYPE["f32"])), 8) == 0
    # int8 pools (hp_paged_attention_q8) need the same workspace as 16-bit ones
    assert L.hp_attention_workspace_bytes(ctypes.byref(desc(dtype=hp.DTYPE["i8"])), 8) == \
        L.hp_attention_workspace_bytes(ctypes.byref(f), 8)
    assert L.hp_attention_workspace_bytes(ctypes.byref(f), 6) == 0
    for hq in (4, 12, 20, 28, 44, 256):                            # any group size is accepted
        assert L.hp_attention_workspace_bytes(ctypes.byref(f), hq) > 0
    a = L.hp_attention_workspace_bytes(ctypes.byref(f), 8)
    b = L.hp_attention_workspace_bytes(ctypes.byref(f), 16)
    assert 0 < a < b
    big = desc(total_tokens=1 << 20, num_pages=1 << 17)
    assert L.hp_attention_workspace_bytes(ctypes.byref(big), 8) > a


KS = ALIGNED + 0x60000000   # K scales
VS = ALIGNED + 0x70000000   # V scales


def attn8(d, v=ALIGNED + 0x40000000, vs=VS, q=ALIGNED + 0x50000000, hq=8, out=OUT, ws=None,
          n=None, flags=0):
    if ws is None:
        ws = ALIGNED + 0x200000000
        n = 1 << 30 if n is None else n
    return L.hp_paged_attention_q8(ctypes.byref(d) if d is not None else None, v, vs, q, hq,
                                   0.125, out, hp.DTYPE["f32"], ws, n or 0, flags, None)


def test_attention_plan_rejections():
    f = desc()
    need = L.hp_attention_workspace_bytes(ctypes.byref(f), 8)
    ws = ALIGNED + 0x200000000
    plan = lambda d, hq=8, w=ws, n=need, flags=0: L.hp_attention_plan(
        ctypes.byref(d) if d is not None else None, hq, w, n, flags, None)
    assert plan(desc(num_seqs=0, num_block_entries=0, total_tokens=0)) == S["HP_OK"]
    assert plan(None) == S["HP_ERR_NULL"]
    assert plan(desc(dtype=hp.DTYPE["f32"])) == S["HP_ERR_DTYPE"]
    assert plan(f, hq=6) == S["HP_ERR_ARG"]
    assert plan(f, flags=hp.HP_FLAG_PLANNED) == S["HP_ERR_ARG"]
    assert plan(f, flags=hp.HP_FLAG_GATED) == S["HP_ERR_ARG"]
    assert plan(f, n=need - 1) == S["HP_ERR_WORKSPACE"]
    assert plan(f, w=None, n=0) == S["HP_ERR_WORKSPACE"]
    assert plan(f, w=ws + 64) == S["HP_ERR_ALIGN"]
    # the attention calls take the flag
    assert attn(desc(num_seqs=0, num_block_entries=0, total_tokens=0),
                flags=hp.HP_FLAG_PLANNED) == S["HP_OK"]
    assert attn8(desc(dtype=hp.DTYPE["i8"], num_seqs=0, num_block_entries=0, total_tokens=0),
                 flags=hp.HP_FLAG_PLANNED) == S["HP_OK"]


def test_attention_q8_rejections():
    f = desc(dtype=hp.DTYPE["i8"], scales=KS)
    assert attn8(desc(dtype=hp.DTYPE["i8"], num_seqs=0, num_block_entries=0,
                      total_tokens=0)) == S["HP_OK"]             # no work, scales not needed
    assert attn8(None) == S["HP_ERR_NULL"]
    assert attn8(desc(dtype=hp.DTYPE["f16"], scales=KS)) == S["HP_ERR_DTYPE"]
    assert attn8(desc(dtype=hp.DTYPE["bf16"], scales=KS)) == S["HP_ERR_DTYPE"]
    assert attn8(desc(dtype=hp.DTYPE["u8"], scales=KS)) == S["HP_ERR_DTYPE"]
    assert attn8(desc(dtype=hp.DTYPE["i8"])) == S["HP_ERR_NULL"]     # no K scales
    assert attn8(f, vs=None) == S["HP_ERR_NULL"]
    assert attn8(f, v=None) == S["HP_ERR_NULL"]
    assert attn8(f, vs=VS + 4) == S["HP_ERR_ALIGN"]
    assert attn8(desc(dtype=hp.DTYPE["i8"], scales=KS + 4)) == S["HP_ERR_ALIGN"]
    assert attn8(f, hq=6) == S["HP_ERR_ARG"]
    assert attn8(f, flags=hp.HP_FLAG_GATED) == S["HP_ERR_ARG"]
    need = L.hp_attention_workspace_bytes(ctypes.byref(f), 8)
    assert attn8(f, n=need - 1) == S["HP_ERR_WORKSPACE"]
    assert attn8(f, out=KS + 64) == S["HP_ERR_ARG"]               # out over the K scales
    assert attn8(f, out=VS) == S["HP_ERR_ARG"]                    # out over the V scales
    assert attn8(f, ws=VS - 256, n=need) == S["HP_ERR_ARG"]       # workspace over the V scales
    assert attn8(f, out=ALIGNED + 64) == S["HP_ERR_ARG"]          # out over the K pool


def sq(d, src=OUT, sdt=None, zp=None, flags=0):
    sdt = hp.DTYPE["f16"] if sdt is None else sdt
    return L.hp_scatter_quant(ctypes.byref(d) if d is not None else None, src, sdt, zp, None,
                              None, 0, flags, None)


def test_scatter_quant_rejections():
    i8 = desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500000)
    u8 = desc(dtype=hp.DTYPE["u8"], scales=ALIGNED + 0x500000)
    ZP = ALIGNED + 0x600000
    assert sq(None) == S["HP_ERR_NULL"]
    assert sq(desc(scales=ALIGNED + 0x500000)) == S["HP_ERR_DTYPE"]   # f16 pool
    assert sq(i8, sdt=hp.DTYPE["i8"]) == S["HP_ERR_DTYPE"]           # int8 source
    assert sq(i8, sdt=hp.DTYPE["f64"]) == S["HP_ERR_DTYPE"]
    assert sq(i8, zp=ZP) == S["HP_ERR_ARG"]                           # symmetric: no zero points
    assert sq(u8) == S["HP_ERR_NULL"]                                 # asymmetric needs them
    assert sq(desc(dtype=hp.DTYPE["i8"])) == S["HP_ERR_NULL"]         # no scales
    assert sq(i8, src=None) == S["HP_ERR_NULL"]
    assert sq(i8, src=OUT + 1) == S["HP_ERR_ALIGN"]
    assert sq(i8, src=OUT + 2, sdt=hp.DTYPE["f32"]) == S["HP_ERR_ALIGN"]
    assert sq(u8, zp=ZP + 8) == S["HP_ERR_ALIGN"]
    assert sq(i8, src=ALIGNED + 0x400) == S["HP_ERR_ARG"]             # source over the pool
    assert sq(i8, src=ALIGNED + 0x500000) == S["HP_ERR_ARG"]          # source over the scales
    assert sq(u8, zp=ALIGNED + 0x500000) == S["HP_ERR_ARG"]           # zero points over scales
    assert sq(u8, zp=ALIGNED) == S["HP_ERR_ARG"]                      # zero points over the pool
    assert sq(i8, flags=hp.HP_FLAG_STREAM) == S["HP_ERR_ARG"]
    assert sq(i8, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    empty = desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500000, num_seqs=0,
                 num_block_entries=0, total_tokens=0)
    assert sq(empty, src=None) == S["HP_OK"]                          # nothing to write


def test_workspace_bytes():
    d = desc()
    assert L.hp_workspace_bytes(ctypes.byref(d)) == 256
    big = desc(num_seqs=5000, num_block_entries=20000, num_pages=20000)
    n = L.hp_workspace_bytes(ctypes.byref(big))
    # validator head + per-sequence offsets (8 + 4 bytes) + chunk totals
    assert n >= 256 + 12 * 5000
    # more sequences than fit in LDS: an unchecked call needs the plan arrays
    assert gather(big) == S["HP_ERR_WORKSPACE"]


def test_empty_batch_and_zero_tokens_enqueue_nothing():
    """[Hurray] Buffer Table note: num_seqs = 0, seq_ptr = [0], block_table
    may be NULL. No work is enqueued, so this runs without a GPU."""
    d = desc(num_seqs=0, num_block_entries=0, block_table=None, seq_lens=None, total_tokens=0)
    assert gather(d, out=None) == S["HP_OK"]
    assert L.hp_scatter(ctypes.byref(d), None, None, None, 0, hp.HP_FLAG_ZERO_TAIL, None) == 0
    z = desc(total_tokens=0)
    assert gather(z, out=None) == S["HP_OK"]


def _arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def test_batch_rejections():
    """Batched calls check every member before enqueuing anything."""
    d = desc()
    P1, P2 = ALIGNED, ALIGNED + 0x10000000          # two distinct 64-byte aligned pools
    O1, O2 = OUT, OUT + 0x10000000
    g = lambda n, pools, outs, flags=0: L.hp_gather_batch(  # noqa: E731
        ctypes.byref(d), n, pools, outs, None, 0, flags, None)
    assert L.hp_gather_batch(None, 2, _arr(P1, P2), _arr(O1, O2), None, 0, 0, None) == S["HP_ERR_NULL"]
    assert g(0, None, None) == S["HP_OK"]                      # nothing to do
    assert g(2, None, _arr(O1, O2)) == S["HP_ERR_NULL"]
    assert g(2, _arr(P1, None), _arr(O1, O2)) == S["HP_ERR_NULL"]
    assert g(2, _arr(P1, P2 + 32), _arr(O1, O2)) == S["HP_ERR_ALIGN"]
    assert g(2, _arr(P1, P2), _arr(O1, O2 + 1)) == S["HP_ERR_ALIGN"]
    assert g(2, _arr(P1, P2), _arr(O1, O1 + 64)) == S["HP_ERR_ARG"]     # outputs overlap
    assert g(2, _arr(P1, P2), _arr(O1, P2 + 256)) == S["HP_ERR_ARG"]    # output inside a pool
    assert g(2, _arr(P1, P2), _arr(O1, O2), flags=16) == S["HP_ERR_ARG"]
    assert g(2, _arr(P1, P2), _arr(O1, O2), flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    bad = desc(rank=2)
    assert L.hp_gather_batch(ctypes.byref(bad), 2, _arr(P1, P2), _arr(O1, O2), None, 0, 0,
                             None) == S["HP_ERR_RANK"]
    sc = lambda pools, srcs, flags=0: L.hp_scatter_batch(  # noqa: E731
        ctypes.byref(d), 2, pools, srcs, None, None, 0, flags, None)
    assert sc(_arr(P1, P1 + 64), _arr(O1, O2)) == S["HP_ERR_ARG"]      # written pools overlap
    assert sc(_arr(P1, P2), _arr(O1, O2), hp.HP_FLAG_STREAM) == S["HP_ERR_ARG"]
    q = desc(dtype=hp.DTYPE["i8"])
    S1, S2 = ALIGNED + 0x20000000, ALIGNED + 0x30000000
    dq = lambda scales, od=hp.DTYPE["bf16"], dd=q: L.hp_gather_dequant_batch(  # noqa: E731
        ctypes.byref(dd), 2, _arr(P1, P2), scales, _arr(O1, O2), od, None, 0, 0, None)
    assert dq(None) == S["HP_ERR_NULL"]
    assert dq(_arr(S1, None)) == S["HP_ERR_NULL"]
    assert dq(_arr(S1, S2 + 4)) == S["HP_ERR_ALIGN"]
    assert dq(_arr(S1, S2), od=hp.DTYPE["f16"]) == S["HP_ERR_DTYPE"]
    assert dq(_arr(S1, S2), dd=d) == S["HP_ERR_DTYPE"]


def test_batch_empty_batch_enqueues_nothing():
    d = desc(num_seqs=0, num_block_entries=0, block_table=None, seq_lens=None, total_tokens=0)
    assert L.hp_gather_batch(ctypes.byref(d), 2, _arr(ALIGNED, ALIGNED + 0x10000000),
                             _arr(None, None), None, 0, 0, None) == S["HP_OK"]


def test_copy_pages_rejections():
    d = desc()
    src, dst = ALIGNED + 0x40000000, ALIGNED + 0x40001000
    cp = lambda dd, s_, d_, n, flags=0, ws=None, wn=0: L.hp_copy_pages(  # noqa: E731
        ctypes.byref(dd) if dd is not None else None, s_, d_, n, ws, wn, flags, None)
    assert cp(None, src, dst, 4) == S["HP_ERR_NULL"]
    assert cp(desc(rank=2), src, dst, 4) == S["HP_ERR_RANK"]
    assert cp(d, src, dst, 0) == S["HP_OK"]                       # nothing to copy
    assert cp(d, None, dst, 4) == S["HP_ERR_NULL"]
    assert cp(d, src + 2, dst, 4) == S["HP_ERR_ALIGN"]            # u32 page IDs
    assert cp(d, src, dst, 4, flags=2) == S["HP_ERR_ARG"]         # scatter-only flag
    assert cp(d, src, dst, 4, flags=hp.HP_FLAG_CHECKED) == S["HP_ERR_WORKSPACE"]
    assert cp(desc(page_pool=ALIGNED + 16), src, dst, 4) == S["HP_ERR_ALIGN"]
    P1, P2 = ALIGNED, ALIGNED + 0x10000000
    cb = lambda pools, n=2: L.hp_copy_pages_batch(  # noqa: E731
        ctypes.byref(d), n, pools, None, src, dst, 4, None, 0, 0, None)
    assert cb(None) == S["HP_ERR_NULL"]
    assert cb(_arr(P1, P1 + 64)) == S["HP_ERR_ARG"]               # written pools overlap
    assert cb(_arr(P1, None)) == S["HP_ERR_NULL"]
    assert cb(_arr(P1, P2 + 8)) == S["HP_ERR_ALIGN"]
    assert cb(_arr(P1, P2), n=0) == S["HP_OK"]


def test_descriptor_handle_keeps_tensors_alive():
    """The handle from with_tokens() carries raw pointers into the descriptor's
    tensors, so it keeps them alive even when the Descriptor object and every
    other reference are gone (a freed index tensor would be handed to the next
    allocation, and its pointer would then name foreign data)."""
    import gc
    import weakref

    import numpy as np
    import torch

    def idx(a):
        return torch.from_numpy(np.asarray(a, np.uint32).view(np.int32).copy())

    pool = torch.zeros((4, 16, 2, 8), dtype=torch.float16)
    bt = idx([0, 1])
    alive = weakref.ref(bt)
    handle = hp.Descriptor(pool, bt, idx([0, 2]), idx([20])).with_tokens(20)
    del bt
    gc.collect()
    assert alive() is not None
    del handle
    gc.collect()
    assert alive() is None


def test_gated_and_async_validation_rejections():
    """The gated form needs the workspace that holds the verdict, and is not
    combined with the synchronous check; hp_validate_async checks the
    descriptor on the host like hp_validate."""
    d = desc()
    G, C = hp.HP_FLAG_GATED, hp.HP_FLAG_CHECKED
    assert gather(d, flags=G) == S["HP_ERR_WORKSPACE"]
    assert gather(d, ws=OUT + 0x100000, n=255, flags=G) == S["HP_ERR_WORKSPACE"]
    assert gather(d, ws=OUT + 0x100004, n=4096, flags=G) == S["HP_ERR_ALIGN"]
    assert gather(d, ws=OUT + 0x100000, n=4096, flags=G | C) == S["HP_ERR_ARG"]
    assert L.hp_scatter(ctypes.byref(d), OUT, None, None, 0, G, None) == S["HP_ERR_WORKSPACE"]
    q = desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500000)
    assert L.hp_gather_dequant(ctypes.byref(q), OUT, hp.DTYPE["bf16"], None, 0, G, None) == \
        S["HP_ERR_WORKSPACE"]
    va = L.hp_validate_async
    assert va(None, None, OUT, 4096, None) == S["HP_ERR_NULL"]
    assert va(ctypes.byref(desc(rank=2)), None, OUT, 4096, None) == S["HP_ERR_RANK"]
    assert va(ctypes.byref(d), None, None, 0, None) == S["HP_ERR_WORKSPACE"]
    assert va(ctypes.byref(d), None, OUT, 255, None) == S["HP_ERR_WORKSPACE"]
    assert va(ctypes.byref(d), ALIGNED + 0x400002, OUT, 4096, None) == S["HP_ERR_ALIGN"]
    # attention and page copies are not gated
    assert L.hp_copy_pages(ctypes.byref(d), ALIGNED, ALIGNED, 1, OUT, 4096, G, None) == \
        S["HP_ERR_ARG"]


def test_validate_verdict_decoding():
    """hp_validate_verdict reads the two words the device check leaves: the
    smallest failing (check, index) key and the token sum."""
    d = desc()  # total_tokens = 114
    res = hp.HpValidateResult()

    def verdict(key, total):
        words = (ctypes.c_uint64 * 2)(key, total)
        return L.hp_validate_verdict(ctypes.byref(d), words, ctypes.byref(res)), res.index

    ones = (1 << 64) - 1
    assert verdict(ones, 114) == (S["HP_OK"], 0)
    assert verdict(ones, 113) == (S["HP_ERR_TOTAL_TOKENS"], 0)
    assert verdict((1 << 56) | 0, 114) == (S["HP_ERR_SEQPTR_FIRST"], 0)
    assert verdict((2 << 56) | 3, 114) == (S["HP_ERR_SEQPTR_LAST"], 3)
    assert verdict((3 << 56) | 7, 114) == (S["HP_ERR_SEQPTR_ORDER"], 7)
    assert verdict((4 << 56) | 9, 0) == (S["HP_ERR_PAGE_RANGE"], 9)
    assert verdict((5 << 56) | 2, 114) == (S["HP_ERR_SEQ_LEN"], 2)
    assert L.hp_validate_verdict(ctypes.byref(d), None, ctypes.byref(res)) == S["HP_ERR_NULL"]


def test_gather_static_rejections():
    """The allocation-free gather checks everything on the host before it
    touches the device: its size limit, the gated flag (the verdict it would
    read lives in a caller's workspace), and what hp_gather rejects."""
    gs = L.hp_gather_static
    d = desc()
    assert gs(None, OUT, 0, None) == S["HP_ERR_NULL"]
    assert gs(ctypes.byref(desc(rank=2)), OUT, 0, None) == S["HP_ERR_RANK"]
    assert gs(ctypes.byref(d), OUT, hp.HP_FLAG_GATED, None) == S["HP_ERR_ARG"]
    assert gs(ctypes.byref(d), OUT, hp.HP_FLAG_ZERO_TAIL, None) == S["HP_ERR_ARG"]
    assert gs(ctypes.byref(d), OUT + 1, 0, None) == S["HP_ERR_ALIGN"]
    assert gs(ctypes.byref(d), ALIGNED + 64, 0, None) == S["HP_ERR_ARG"]      # overlaps the pool
    big = desc(num_seqs=(1 << 18) + 1, num_block_entries=1 << 19, num_pages=1 << 19)
    assert gs(ctypes.byref(big), OUT, 0, None) == S["HP_ERR_WORKSPACE"]
    empty = desc(num_seqs=0, num_block_entries=0, block_table=None, seq_lens=None,
                 total_tokens=0)
    assert gs(ctypes.byref(empty), None, 0, None) == S["HP_OK"]             # nothing to move


def test_disjoint_writes_rejections():
    """The write-disjointness check is part of the synchronous checked form
    only, on the scatter calls, and needs the bitmaps' workspace; all of this
    is decided on the host before the device is touched."""
    d = desc()
    C, D, G, Z = hp.HP_FLAG_CHECKED, hp.HP_FLAG_DISJOINT, hp.HP_FLAG_GATED, hp.HP_FLAG_ZERO_TAIL
    need = L.hp_disjoint_workspace_bytes(ctypes.byref(d))
    # 512 + two bitmaps of 20 pages x 16 slots (10 words each)
    assert need == 512 + 8 * 10
    assert L.hp_disjoint_workspace_bytes(None) == 0
    assert L.hp_disjoint_workspace_bytes(ctypes.byref(desc(rank=2))) == 0
    big = desc(num_seqs=5000, num_block_entries=20000, num_pages=20000)
    assert L.hp_disjoint_workspace_bytes(ctypes.byref(big)) >= \
        L.hp_workspace_bytes(ctypes.byref(big))
    ws = OUT + 0x100000
    sc = L.hp_scatter
    assert sc(ctypes.byref(d), OUT, None, ws, 4096, D, None) == S["HP_ERR_ARG"]        # unchecked
    assert sc(ctypes.byref(d), OUT, None, ws, 4096, D | G, None) == S["HP_ERR_ARG"]    # gated
    assert sc(ctypes.byref(d), OUT, None, ws, need - 8, C | D, None) == S["HP_ERR_WORKSPACE"]
    assert sc(ctypes.byref(d), OUT, None, ws, 256, C | D | Z, None) == S["HP_ERR_WORKSPACE"]
    assert gather(d, ws=ws, n=4096, flags=C | D) == S["HP_ERR_ARG"]                     # not a scatter
    q = desc(dtype=hp.DTYPE["i8"], scales=ALIGNED + 0x500000)
    assert L.hp_gather_dequant(ctypes.byref(q), OUT, hp.DTYPE["bf16"], ws, 4096, C | D,
                               None) == S["HP_ERR_ARG"]
    assert sq(q, flags=D) == S["HP_ERR_ARG"]
    vw = L.hp_validate_writes
    res = hp.HpValidateResult()
    assert vw(None, None, 0, ws, need, ctypes.byref(res), None) == S["HP_ERR_NULL"]
    assert vw(ctypes.byref(d), None, C, ws, need, ctypes.byref(res), None) == S["HP_ERR_ARG"]
    assert res.code == S["HP_ERR_ARG"]
    assert vw(ctypes.byref(d), None, Z, ws, need - 1, None, None) == S["HP_ERR_WORKSPACE"]
    assert vw(ctypes.byref(d), None, 0, ws + 4, need, None, None) == S["HP_ERR_ALIGN"]
    assert vw(ctypes.byref(d), ALIGNED + 0x400002, 0, ws, need, None, None) == S["HP_ERR_ALIGN"]
    assert vw(ctypes.byref(desc(paged_axis=1)), None, 0, ws, need, None, None) == \
        S["HP_ERR_PAGED_AXIS"]
