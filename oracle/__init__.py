"""CPU oracle for the block-paged KV layout: numpy front end to liboracle.so.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the GPU library (``block_table_gather_amd``) and neither imports the
other. Nothing here may serve as a fallback for the GPU path.

Every function takes numpy arrays, widens index arrays to uint64 (lossless)
and calls the plain C element loops of ``oracle.c``, which cite the pages:

* [Hurray] "Block-Paged Layout -- Hurray Format Specification"
* [Rust20] "Keep token order across cache pages"
* [Day51]  "Visualize PagedAttention block layout"

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py``, ``tests/test_oracle_cross.py`` and
``tests/test_oracle_attention.py``.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# HP_ORACLE_LIB names another build of the same source (the sanitizer test's)
LIB_PATH = os.environ.get("HP_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

# Oracle check outcomes (oracle.h, enum oracle_check), by name.
CHECKS = {
    0: "valid",
    1: "rank",
    2: "paged_axis",
    3: "seq_ptr_first",
    4: "seq_ptr_last",
    5: "seq_ptr_order",
    6: "page_range",
    7: "seq_len",
    8: "total_tokens",
}

_lib = None
_u64p = ctypes.POINTER(ctypes.c_uint64)
_vp = ctypes.c_void_p
_u64 = ctypes.c_uint64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_element_index.restype = _u64
    lib.oracle_element_index.argtypes = [_vp, _vp] + [_u64] * 9
    lib.oracle_validate.restype = ctypes.c_int
    lib.oracle_validate.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _u64, _u64, _vp,
                                    _u64, _vp, _u64, _vp, _vp, _u64, _vp]
    lib.oracle_disjoint_writes.restype = ctypes.c_int
    lib.oracle_disjoint_writes.argtypes = [_u64, _u64, _vp, _vp, _u64, _vp, _vp, ctypes.c_int,
                                           _vp]
    lib.oracle_gather.restype = None
    lib.oracle_gather.argtypes = [_vp, _u64, _u64, _u64, _u64, _vp, _vp, _vp, _u64,
                                  _vp, _vp]
    lib.oracle_gather_rows.restype = _u64
    lib.oracle_gather_rows.argtypes = [_vp, _u64, _u64, _u64, _u64, _vp, _vp, _vp,
                                       _u64, _vp, _u64, _vp]
    lib.oracle_scatter.restype = None
    lib.oracle_scatter.argtypes = [_vp, _u64, _u64, _u64, _u64, _vp, _vp, _vp, _vp,
                                   _u64, _vp, ctypes.c_int]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_bf16_rne_array.argtypes = [_vp, _u64, _vp]
    lib.oracle_gather_dequant.restype = None
    lib.oracle_gather_dequant.argtypes = [_vp, _vp, _u64, _u64, _u64, _vp, _vp, _vp,
                                          _u64, _vp]
    lib.oracle_gather_dequant_rows.restype = _u64
    lib.oracle_gather_dequant_rows.argtypes = [_vp, _vp, _u64, _u64, _u64, _vp, _vp,
                                               _vp, _u64, _vp, _u64, _vp]
    lib.oracle_quant_accepts.restype = ctypes.c_int
    lib.oracle_quant_accepts.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _u64, _u64]
    lib.oracle_gather_dequant_scheme.restype = None
    lib.oracle_gather_dequant_scheme.argtypes = [_vp, ctypes.c_int, ctypes.c_uint32,
                                                 ctypes.c_uint32, _vp, _vp, _u64, _u64, _u64,
                                                 _vp, _vp, _vp, _u64, _vp]
    lib.oracle_copy_pages.restype = None
    lib.oracle_copy_pages.argtypes = [_vp, _u64, _u64, _u64, _u64, _vp, _vp, _vp, _u64]
    lib.oracle_payload.restype = ctypes.c_int
    lib.oracle_payload.argtypes = [_u64] * 7 + [_vp]
    lib.oracle_quantize_row.restype = None
    lib.oracle_quantize_row.argtypes = [_vp, _u64, ctypes.c_int, _vp, _vp, _vp]
    lib.oracle_scatter_quant.restype = None
    lib.oracle_scatter_quant.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_uint32, _u64, _u64, _u64,
                                         _vp, _vp, _vp, _vp, _u64, ctypes.c_int]
    lib.oracle_decode.restype = None
    lib.oracle_decode.argtypes = [ctypes.c_uint32, _vp, _u64, _vp]
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [_vp, _vp, _vp, ctypes.c_uint32, _u64, _u64, _u64,
                                           _u64, ctypes.c_double, _vp, _vp, _vp, _u64, _vp]
    lib.oracle_paged_attention_q8.restype = ctypes.c_int
    lib.oracle_paged_attention_q8.argtypes = [_vp, _vp, _vp, _vp, _vp, _u64, _u64, _u64, _u64,
                                              ctypes.c_double, _vp, _vp, _vp, _u64, _vp]
    _lib = lib
    return lib


def _idx(a):
    """Index array as contiguous uint64 (kept alive by the caller)."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint64))


def _ptr(a):
    return None if a is None else a.ctypes.data


def element_index(block_table, seq_ptr, s, t, h, d, page_size, strides):
    """[Hurray] Element Lookup with explicit (page, slot, head, dim) strides."""
    lib = _load()
    bt, sp = _idx(block_table), _idx(seq_ptr)
    return int(lib.oracle_element_index(_ptr(bt), _ptr(sp), s, t, h, d, page_size,
                                        *strides))


def validate(*, rank, paged_axis, num_pages, page_size, block_table, seq_ptr,
             seq_lens, total_tokens, seq_start=None):
    """First failing storage check, as (name, index); ("valid", 0) if none."""
    lib = _load()
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    ss = None if seq_start is None else _idx(seq_start)
    num_seqs = len(sp) - 1
    assert len(sl) == num_seqs and (ss is None or len(ss) == num_seqs)
    index = np.zeros(1, dtype=np.uint64)
    code = lib.oracle_validate(rank, paged_axis, num_pages, page_size,
                               _ptr(bt) if len(bt) else None, len(bt), _ptr(sp),
                               num_seqs, _ptr(sl), _ptr(ss), total_tokens,
                               _ptr(index))
    return CHECKS[code], int(index[0])


def disjoint_writes(*, num_pages, page_size, block_table, seq_ptr, seq_lens, seq_start=None,
                    zero_tail=False):
    """Whether a scatter's written slots are pairwise distinct: None if so,
    else the smallest sequence index one of whose written slots is written
    more than once. The descriptor must be valid."""
    lib = _load()
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    ss = None if seq_start is None else _idx(seq_start)
    num_seqs = len(sp) - 1
    assert len(sl) == num_seqs and (ss is None or len(ss) == num_seqs)
    first = np.zeros(1, dtype=np.uint64)
    found = lib.oracle_disjoint_writes(num_pages, page_size, _ptr(bt) if len(bt) else None,
                                       _ptr(sp), num_seqs, _ptr(sl), _ptr(ss),
                                       int(bool(zero_tail)), _ptr(first))
    return int(first[0]) if found else None


def _pool_geometry(pool, page_size, num_heads, head_dim):
    pool = np.ascontiguousarray(pool)
    assert pool.size % (page_size * num_heads * head_dim) == 0
    return pool, pool.dtype.itemsize


def gather(pool, *, page_size, num_heads, head_dim, block_table, seq_ptr, seq_lens,
           mark_reads=False):
    """Logical [T, H, D] tensor in the pool's dtype (bit copy).

    With mark_reads, also returns a uint8 array over the pool's slots that is 1
    where the gather read a slot."""
    lib = _load()
    pool, eb = _pool_geometry(pool, page_size, num_heads, head_dim)
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    total = int(sl.sum()) if len(sl) else 0
    out = np.empty((total, num_heads, head_dim), dtype=pool.dtype)
    mark = np.zeros(pool.size // (num_heads * head_dim), dtype=np.uint8) \
        if mark_reads else None
    lib.oracle_gather(_ptr(pool), eb, page_size, num_heads, head_dim,
                      _ptr(bt) if len(bt) else None, _ptr(sp), _ptr(sl) if len(sl) else None,
                      len(sl), _ptr(out) if out.size else None, _ptr(mark))
    return (out, mark) if mark_reads else out


def gather_rows(pool, rows, *, page_size, num_heads, head_dim, block_table, seq_ptr,
                seq_lens):
    """Rows `rows` of the logical tensor, computed one by one."""
    lib = _load()
    pool, eb = _pool_geometry(pool, page_size, num_heads, head_dim)
    bt, sp, sl, rw = _idx(block_table), _idx(seq_ptr), _idx(seq_lens), _idx(rows)
    out = np.zeros((len(rw), num_heads, head_dim), dtype=pool.dtype)
    missing = lib.oracle_gather_rows(_ptr(pool), eb, page_size, num_heads, head_dim,
                                     _ptr(bt), _ptr(sp), _ptr(sl), len(sl), _ptr(rw),
                                     len(rw), _ptr(out))
    assert missing == 0, f"{missing} rows past the logical total"
    return out


def scatter(pool, src, *, page_size, num_heads, head_dim, block_table, seq_ptr,
            seq_lens, seq_start=None, zero_tail=False, in_place=False):
    """Returns a copy of `pool` with the rows of `src` written into their slots
    (with in_place, writes into `pool` itself, which must be contiguous)."""
    lib = _load()
    if in_place:
        assert pool.flags["C_CONTIGUOUS"]
        result, eb = pool, pool.dtype.itemsize
    else:
        pool, eb = _pool_geometry(pool, page_size, num_heads, head_dim)
        result = pool.copy()
    src = np.ascontiguousarray(src)
    assert src.dtype.itemsize == eb
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    ss = None if seq_start is None else _idx(seq_start)
    lib.oracle_scatter(_ptr(result), eb, page_size, num_heads, head_dim,
                       _ptr(bt) if len(bt) else None, _ptr(sp),
                       _ptr(sl) if len(sl) else None, _ptr(ss) if ss is not None and len(ss) else None,
                       len(sl), _ptr(src) if src.size else None, int(bool(zero_tail)))
    return result


def bf16_rne(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        lib.oracle_bf16_rne_array(_ptr(x), x.size, _ptr(out))
    return out


def gather_dequant(pool, scales, *, page_size, num_heads, head_dim, block_table,
                   seq_ptr, seq_lens):
    """int8 pool + per-slot fp32 scales -> bf16 bit patterns [T, H, D] (uint16)."""
    lib = _load()
    pool = np.ascontiguousarray(pool, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    total = int(sl.sum()) if len(sl) else 0
    out = np.empty((total, num_heads, head_dim), dtype=np.uint16)
    lib.oracle_gather_dequant(_ptr(pool), _ptr(scales), page_size, num_heads, head_dim,
                              _ptr(bt) if len(bt) else None, _ptr(sp),
                              _ptr(sl) if len(sl) else None, len(sl),
                              _ptr(out) if out.size else None)
    return out


def gather_dequant_rows(pool, scales, rows, *, page_size, num_heads, head_dim,
                        block_table, seq_ptr, seq_lens):
    lib = _load()
    pool = np.ascontiguousarray(pool, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    bt, sp, sl, rw = _idx(block_table), _idx(seq_ptr), _idx(seq_lens), _idx(rows)
    out = np.zeros((len(rw), num_heads, head_dim), dtype=np.uint16)
    missing = lib.oracle_gather_dequant_rows(_ptr(pool), _ptr(scales), page_size,
                                             num_heads, head_dim, _ptr(bt), _ptr(sp),
                                             _ptr(sl), len(sl), _ptr(rw), len(rw),
                                             _ptr(out))
    assert missing == 0
    return out


SCHEMES = {"per_tensor": 0x01, "per_channel": 0x02, "per_block_affine": 0x03}


def quant_accepts(scheme, axis, block_size, page_size):
    """[Hurray] Per-scheme composition: may a reader accept this scheme?"""
    return bool(_load().oracle_quant_accepts(SCHEMES[scheme], axis, block_size, page_size))


def gather_dequant_scheme(pool, scheme, axis, scales, zero_points=None, *, page_size,
                          num_heads, head_dim, block_table, seq_ptr, seq_lens):
    """bf16 bits [T, H, D] of bf16(fp32(q - zp) * scale) under `scheme`; the
    pool is int8 or uint8 (its numpy dtype decides), zero points likewise."""
    lib = _load()
    pool = np.ascontiguousarray(pool)
    assert pool.dtype in (np.int8, np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zp = None if zero_points is None else np.ascontiguousarray(zero_points, dtype=pool.dtype)
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    total = int(sl.sum()) if len(sl) else 0
    out = np.empty((total, num_heads, head_dim), dtype=np.uint16)
    lib.oracle_gather_dequant_scheme(_ptr(pool), int(pool.dtype == np.int8), SCHEMES[scheme],
                                     axis, _ptr(scales), _ptr(zp), page_size, num_heads,
                                     head_dim, _ptr(bt) if len(bt) else None, _ptr(sp),
                                     _ptr(sl) if len(sl) else None, len(sl),
                                     _ptr(out) if out.size else None)
    return out


def copy_pages(pool, src_pages, dst_pages, *, page_size, num_heads, head_dim, scales=None):
    """Copy-on-write page copy; returns (new pool, new scales or None)."""
    lib = _load()
    pool, eb = _pool_geometry(pool, page_size, num_heads, head_dim)
    result = pool.copy()
    sc = None if scales is None else np.array(scales, dtype=np.float32, copy=True)
    src, dst = _idx(src_pages), _idx(dst_pages)
    assert len(src) == len(dst)
    lib.oracle_copy_pages(_ptr(result), eb, page_size, num_heads, head_dim, _ptr(sc),
                          _ptr(src) if len(src) else None, _ptr(dst) if len(dst) else None,
                          len(src))
    return result, sc


# Element types of the attention oracle (oracle.h, enum oracle_float_type).
FLOAT_TYPES = {"f16": 3, "bf16": 4, "f32": 5}


def decode(bits, elem_type):
    """Exact float64 values of stored f16 / bf16 (uint16 bit patterns) or f32
    (uint32 bit patterns) elements."""
    bits = np.ascontiguousarray(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    if bits.size:
        _load().oracle_decode(FLOAT_TYPES[elem_type], _ptr(bits), bits.size, _ptr(out))
    return out


def paged_attention(q, k_pool, v_pool, elem_type, *, page_size, num_kv_heads, head_dim,
                    block_table, seq_ptr, seq_lens, scale):
    """Decode attention over the block-paged K/V cache, float64
    [num_seqs, num_q_heads, head_dim]. q: [num_seqs, num_q_heads, head_dim] and
    the pools [num_pages, page_size, num_kv_heads, head_dim], all as bit
    patterns (uint16 for f16/bf16, uint32 for f32) of `elem_type`."""
    lib = _load()
    q = np.ascontiguousarray(q)
    k_pool, v_pool = np.ascontiguousarray(k_pool), np.ascontiguousarray(v_pool)
    assert q.ndim == 3 and q.shape[2] == head_dim
    S, Hq = q.shape[0], q.shape[1]
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    assert len(sp) == S + 1 and len(sl) == S
    out = np.empty((S, Hq, head_dim), dtype=np.float64)
    if S == 0:
        return out
    rc = lib.oracle_paged_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), FLOAT_TYPES[elem_type],
                                    page_size, num_kv_heads, head_dim, Hq, float(scale),
                                    _ptr(bt) if len(bt) else None, _ptr(sp), _ptr(sl), S,
                                    _ptr(out))
    if rc != 0:
        raise ValueError("num_q_heads must be a positive multiple of num_kv_heads")
    return out


def paged_attention_q8(q, k_pool, k_scales, v_pool, v_scales, *, page_size, num_kv_heads,
                       head_dim, block_table, seq_ptr, seq_lens, scale):
    """Decode attention over int8 K/V pools with one float32 scale per slot,
    float64 [num_seqs, num_q_heads, head_dim]: every element's value is its
    code times its slot's scale. q: bfloat16 bit patterns (uint16)
    [num_seqs, num_q_heads, head_dim]; pools int8 [num_pages, page_size,
    num_kv_heads, head_dim]; scales float32 [num_pages * page_size]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_pool = np.ascontiguousarray(k_pool).view(np.int8)
    v_pool = np.ascontiguousarray(v_pool).view(np.int8)
    k_scales = np.ascontiguousarray(k_scales, dtype=np.float32)
    v_scales = np.ascontiguousarray(v_scales, dtype=np.float32)
    assert q.ndim == 3 and q.shape[2] == head_dim
    S, Hq = q.shape[0], q.shape[1]
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    assert len(sp) == S + 1 and len(sl) == S
    assert k_pool.size == v_pool.size and k_scales.size * num_kv_heads * head_dim == k_pool.size
    assert v_scales.size == k_scales.size
    out = np.empty((S, Hq, head_dim), dtype=np.float64)
    if S == 0:
        return out
    rc = lib.oracle_paged_attention_q8(_ptr(q), _ptr(k_pool), _ptr(k_scales), _ptr(v_pool),
                                       _ptr(v_scales), page_size, num_kv_heads, head_dim, Hq,
                                       float(scale), _ptr(bt) if len(bt) else None, _ptr(sp),
                                       _ptr(sl), S, _ptr(out))
    if rc != 0:
        raise ValueError("num_q_heads must be a positive multiple of num_kv_heads")
    return out


def quantize_row(x, asym=False):
    """(codes, scale, zero point) of one row of float32 values (see
    oracle_quantize_row): int8 codes, or uint8 codes and a zero point."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.size, dtype=np.uint8 if asym else np.int8)
    sc = np.zeros(1, dtype=np.float32)
    zp = np.zeros(1, dtype=np.uint8)
    _load().oracle_quantize_row(_ptr(x), x.size, int(asym), _ptr(q), _ptr(sc), _ptr(zp))
    return q, np.float32(sc[0]), (int(zp[0]) if asym else None)


def scatter_quant(pool, scales, src, src_type, *, page_size, num_heads, head_dim, block_table,
                  seq_ptr, seq_lens, seq_start=None, zero_points=None, zero_tail=False):
    """Quantize-on-scatter into copies of pool (int8, or uint8 with
    zero_points), scales (float32 [N*P]) and zero_points (uint8 [N*P]);
    returns (pool, scales, zero_points or None). src: [T, H, D] bit patterns
    of src_type ("f16", "bf16", "f32")."""
    lib = _load()
    pool = np.array(pool, copy=True, order="C")
    assert pool.dtype == (np.uint8 if zero_points is not None else np.int8)
    sc = np.array(scales, dtype=np.float32, copy=True)
    zp = None if zero_points is None else np.array(zero_points, dtype=np.uint8, copy=True)
    src = np.ascontiguousarray(src)
    bt, sp, sl = _idx(block_table), _idx(seq_ptr), _idx(seq_lens)
    ss = None if seq_start is None else _idx(seq_start)
    lib.oracle_scatter_quant(_ptr(pool), _ptr(sc), _ptr(zp), _ptr(src) if src.size else None,
                             FLOAT_TYPES[src_type], page_size, num_heads, head_dim,
                             _ptr(bt) if len(bt) else None, _ptr(sp), _ptr(sl) if len(sl) else None,
                             _ptr(ss), len(sl), int(zero_tail))
    return pool, sc, zp


PAYLOAD_FIELDS = ("reserved_pages", "active_pages", "allocated_slots", "live_slots",
                  "unused_slots", "tail_slots", "inactive_slots", "allocated_bytes",
                  "live_bytes", "unused_bytes", "tail_bytes", "inactive_bytes",
                  "contiguous_slots")


def payload(*, capacity, page_tokens, length, batch, kv_heads, width, elem_bytes=8):
    """[Rust20] payload accounting of one layer's K and V arrays, as a dict."""
    lib = _load()
    out = np.zeros(13, dtype=np.uint64)
    rc = lib.oracle_payload(capacity, page_tokens, length, batch, kv_heads, width,
                            elem_bytes, _ptr(out))
    if rc != 0:
        raise ValueError("invalid payload query")
    return {k: int(v) for k, v in zip(PAYLOAD_FIELDS, out)}
