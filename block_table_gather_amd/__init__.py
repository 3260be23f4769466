"""Block-paged KV gather / scatter / dequant-gather / validate on MI355X.

Thin ctypes binding over ``libhp.so`` (the C ABI declared in
``include/hp.h``). This module only marshals arguments: it reads pointers,
sizes and the current HIP stream from torch tensors and calls the library;
every step of the path runs in the library's HIP kernels. PyTorch is used for
device memory and streams only.

The layout is the one of "Block-Paged Layout -- Hurray Format Specification":
page pool [num_pages, page_size, num_heads, head_dim], a block table of
physical page IDs (uint32 or uint64), CSR offsets ``seq_ptr`` and one token
count per sequence. Importing this package fails if the library was not built
(``python -m block_table_gather_amd.build``); there is no fallback.
"""
import ctypes
import os

# PyTorch ships its own HIP runtime under the same soname (libamdhip64.so.7)
# as the system ROCm one that libhp.so is linked against. Loading torch first
# makes the dynamic linker bind libhp.so to torch's copy, so that one HIP
# runtime serves both (two runtimes in one process cannot share a device).
import torch  # noqa: F401,E402

__all__ = ["Descriptor", "HpError", "gather", "scatter", "gather_dequant", "validate",
           "validate_async", "validate_verdict", "gather_static", "validate_writes",
           "disjoint_workspace_bytes",
           "gather_dequant_q", "QUANT_SCHEME", "paged_attention", "attention_workspace_bytes",
           "scatter_quant",
           "gather_batch", "scatter_batch", "gather_dequant_batch", "copy_pages",
           "copy_pages_batch", "workspace_bytes",
           "status_str", "last_hip_error", "lib", "LIB_PATH", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_table_gather_amd/build.py` "
        "(hipcc, gfx950). There is no fallback implementation.")

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()
    return {os.path.realpath(p) for p in paths}


if len(_hip_runtimes()) > 1:
    raise ImportError(
        "two HIP runtimes are loaded in this process (" + ", ".join(sorted(_hip_runtimes()))
        + "); libhp.so must share torch's: import torch before loading libhp.so")

# Status codes (include/hp.h, enum hp_status).
STATUS = {
    0: "HP_OK", 1: "HP_ERR_NULL", 2: "HP_ERR_ARG", 3: "HP_ERR_RANK", 4: "HP_ERR_PAGED_AXIS",
    5: "HP_ERR_INDEX_TYPE", 6: "HP_ERR_DTYPE", 7: "HP_ERR_ALIGN", 8: "HP_ERR_WORKSPACE",
    9: "HP_ERR_SHARDED", 10: "HP_ERR_QUANT", 16: "HP_ERR_SEQPTR_FIRST", 17: "HP_ERR_SEQPTR_LAST",
    18: "HP_ERR_SEQPTR_ORDER", 19: "HP_ERR_PAGE_RANGE", 20: "HP_ERR_SEQ_LEN",
    21: "HP_ERR_TOTAL_TOKENS", 22: "HP_ERR_WRITE_ALIAS", 32: "HP_ERR_HIP",
}
CODE = {v: k for k, v in STATUS.items()}
HP_INDEX_U32, HP_INDEX_U64 = 0x00, 0x01
DTYPE = {"i8": 1, "u8": 2, "f16": 3, "bf16": 4, "f32": 5, "f64": 6}
HP_FLAG_CHECKED, HP_FLAG_ZERO_TAIL, HP_FLAG_STREAM, HP_FLAG_GATED = 1, 2, 4, 8
HP_FLAG_DISJOINT = 16
HP_FLAG_PLANNED = 32
# Quantization scheme tags (include/hp.h, HP_QUANT_*).
QUANT_SCHEME = {"per_tensor": 0x01, "per_channel": 0x02, "per_block_affine": 0x03}


class HpQuant(ctypes.Structure):
    """Mirror of ``hp_quant`` (include/hp.h)."""
    _fields_ = [
        ("scheme", ctypes.c_uint32), ("axis", ctypes.c_uint32),
        ("block_size", ctypes.c_uint64),
        ("scales", ctypes.c_void_p), ("zero_points", ctypes.c_void_p),
    ]


class HpDesc(ctypes.Structure):
    """Mirror of ``hp_desc`` (include/hp.h)."""
    _fields_ = [
        ("rank", ctypes.c_uint32), ("paged_axis", ctypes.c_uint32),
        ("index_type", ctypes.c_uint32), ("dtype", ctypes.c_uint32),
        ("page_size", ctypes.c_uint32), ("num_heads", ctypes.c_uint32),
        ("head_dim", ctypes.c_uint32), ("has_shard", ctypes.c_uint32),
        ("kv_role", ctypes.c_uint32), ("layer_index", ctypes.c_uint32),
        ("byte_offset", ctypes.c_uint64), ("num_pages", ctypes.c_uint64),
        ("num_seqs", ctypes.c_uint64), ("num_block_entries", ctypes.c_uint64),
        ("total_tokens", ctypes.c_uint64),
        ("page_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("seq_ptr", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
    ]


class HpValidateResult(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("reserved", ctypes.c_uint32),
                ("index", ctypes.c_uint64)]


_P = ctypes.POINTER(HpDesc)
_vp, _sz, _u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32
_lib.hp_workspace_bytes.restype = _sz
_lib.hp_workspace_bytes.argtypes = [_P]
_lib.hp_validate.restype = ctypes.c_int
_lib.hp_validate.argtypes = [_P, _vp, _vp, _sz, ctypes.POINTER(HpValidateResult), _vp]
_lib.hp_validate_async.restype = ctypes.c_int
_lib.hp_validate_async.argtypes = [_P, _vp, _vp, _sz, _vp]
_lib.hp_validate_writes.restype = ctypes.c_int
_lib.hp_validate_writes.argtypes = [_P, _vp, _u32, _vp, _sz, ctypes.POINTER(HpValidateResult),
                                    _vp]
_lib.hp_disjoint_workspace_bytes.restype = _sz
_lib.hp_disjoint_workspace_bytes.argtypes = [_P]
_lib.hp_validate_verdict.restype = ctypes.c_int
_lib.hp_validate_verdict.argtypes = [_P, _vp, ctypes.POINTER(HpValidateResult)]
_lib.hp_gather_static.restype = ctypes.c_int
_lib.hp_gather_static.argtypes = [_P, _vp, _u32, _vp]
_lib.hp_gather.restype = ctypes.c_int
_lib.hp_gather.argtypes = [_P, _vp, _vp, _sz, _u32, _vp]
_lib.hp_scatter.restype = ctypes.c_int
_lib.hp_scatter.argtypes = [_P, _vp, _vp, _vp, _sz, _u32, _vp]
_lib.hp_gather_dequant.restype = ctypes.c_int
_lib.hp_gather_dequant.argtypes = [_P, _vp, _u32, _vp, _sz, _u32, _vp]
_lib.hp_gather_dequant_q.restype = ctypes.c_int
_lib.hp_gather_dequant_q.argtypes = [_P, ctypes.POINTER(HpQuant), _vp, _u32, _vp, _sz, _u32,
                                     _vp]
_lib.hp_scatter_quant.restype = ctypes.c_int
_lib.hp_scatter_quant.argtypes = [_P, _vp, _u32, _vp, _vp, _vp, _sz, _u32, _vp]
_lib.hp_paged_attention.restype = ctypes.c_int
_lib.hp_paged_attention.argtypes = [_P, _vp, _vp, _u32, ctypes.c_float, _vp, _u32, _vp, _sz,
                                    _u32, _vp]
_lib.hp_paged_attention_q8.restype = ctypes.c_int
_lib.hp_paged_attention_q8.argtypes = [_P, _vp, _vp, _vp, _u32, ctypes.c_float, _vp, _u32, _vp,
                                       _sz, _u32, _vp]
_lib.hp_attention_workspace_bytes.restype = _sz
_lib.hp_attention_workspace_bytes.argtypes = [_P, _u32]
_lib.hp_attention_plan.restype = ctypes.c_int
_lib.hp_attention_plan.argtypes = [_P, _u32, _vp, _sz, _u32, _vp]
_lib.hp_status_str.restype = ctypes.c_char_p
_lib.hp_status_str.argtypes = [ctypes.c_int]
_lib.hp_last_hip_error.restype = ctypes.c_char_p
_lib.hp_last_hip_error.argtypes = []
_lib.hp_gather_batch.restype = ctypes.c_int
_lib.hp_gather_batch.argtypes = [_P, _u32, _vp, _vp, _vp, _sz, _u32, _vp]
_lib.hp_scatter_batch.restype = ctypes.c_int
_lib.hp_scatter_batch.argtypes = [_P, _u32, _vp, _vp, _vp, _vp, _sz, _u32, _vp]
_lib.hp_copy_pages.restype = ctypes.c_int
_lib.hp_copy_pages.argtypes = [_P, _vp, _vp, ctypes.c_uint64, _vp, _sz, _u32, _vp]
_lib.hp_copy_pages_batch.restype = ctypes.c_int
_lib.hp_copy_pages_batch.argtypes = [_P, _u32, _vp, _vp, _vp, _vp, ctypes.c_uint64, _vp, _sz,
                                     _u32, _vp]
_lib.hp_gather_dequant_batch.restype = ctypes.c_int
_lib.hp_gather_dequant_batch.argtypes = [_P, _u32, _vp, _vp, _vp, _u32, _vp, _sz, _u32, _vp]


def lib():
    """The loaded ctypes library (raw C ABI)."""
    return _lib


def status_str(code):
    return _lib.hp_status_str(int(code)).decode()


def last_hip_error():
    """HIP error name behind this thread's last HP_ERR_HIP."""
    return _lib.hp_last_hip_error().decode()


class HpError(RuntimeError):
    def __init__(self, code, where=""):
        self.code = int(code)
        self.name = STATUS.get(self.code, str(code))
        msg = status_str(code)
        if self.name == "HP_ERR_HIP":
            msg += f" ({last_hip_error()})"
        super().__init__(f"{where}: {msg}" if where else msg)


def _check(code, where):
    if code != 0:
        raise HpError(code, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _torch():
    return torch


def _dtype_code(t):
    torch = _torch()
    table = {torch.int8: "i8", torch.uint8: "u8", torch.float16: "f16",
             torch.bfloat16: "bf16", torch.float32: "f32", torch.float64: "f64"}
    if t.dtype not in table:
        raise TypeError(f"unsupported page_pool dtype {t.dtype}")
    return DTYPE[table[t.dtype]]


def _index_code(t):
    torch = _torch()
    if t.element_size() == 4 and t.dtype in (torch.int32, getattr(torch, "uint32", None)):
        return HP_INDEX_U32
    if t.element_size() == 8 and t.dtype in (torch.int64, getattr(torch, "uint64", None)):
        return HP_INDEX_U64
    raise TypeError(f"index tensors must be 32- or 64-bit integers, got {t.dtype}")


class Descriptor:
    """A block-paged descriptor over device tensors (kept alive here).

    page_pool: [num_pages, page_size, num_heads, head_dim] tensor (or any
    contiguous tensor of that many elements; then pass the geometry).
    block_table / seq_ptr / seq_lens: int32 (uint32 semantics) or int64
    tensors, all of the same width. scales: float32 [num_pages*page_size] or
    None. The fields rank / paged_axis / byte_offset / has_shard default to
    the only values the layout admits and exist so that a foreign descriptor
    can be passed through unchanged and rejected by the library.
    """

    def __init__(self, page_pool, block_table, seq_ptr, seq_lens, *, page_size=None,
                 num_heads=None, head_dim=None, num_pages=None, scales=None, rank=3,
                 paged_axis=0, byte_offset=0, has_shard=0, kv_role=0, layer_index=0,
                 index_type=None, dtype=None, num_block_entries=None):
        if page_pool.dim() == 4:
            n, p, h, d = page_pool.shape
        else:
            n = p = h = d = None
        self.page_pool, self.block_table, self.seq_ptr = page_pool, block_table, seq_ptr
        self.seq_lens, self.scales = seq_lens, scales
        self.c = HpDesc()
        c = self.c
        # The struct holds raw device pointers into these tensors; the
        # reference from the struct back to this object keeps them alive for
        # as long as any handle from with_tokens() exists.
        c._owner = self
        c.rank, c.paged_axis = rank, paged_axis
        c.index_type = _index_code(seq_ptr) if index_type is None else index_type
        c.dtype = _dtype_code(page_pool) if dtype is None else dtype
        c.page_size = page_size if page_size is not None else p
        c.num_heads = num_heads if num_heads is not None else h
        c.head_dim = head_dim if head_dim is not None else d
        c.has_shard, c.kv_role, c.layer_index = has_shard, kv_role, layer_index
        c.byte_offset = byte_offset
        c.num_pages = num_pages if num_pages is not None else n
        c.num_seqs = seq_ptr.numel() - 1
        c.num_block_entries = (block_table.numel() if block_table is not None else 0) \
            if num_block_entries is None else num_block_entries
        c.total_tokens = 0
        c.page_pool = _ptr(page_pool)
        c.block_table = _ptr(block_table) if block_table is not None and block_table.numel() else None
        c.seq_ptr = _ptr(seq_ptr)
        c.seq_lens = _ptr(seq_lens) if seq_lens is not None and seq_lens.numel() else None
        c.scales = _ptr(scales)

    @property
    def device(self):
        return self.seq_ptr.device

    def with_tokens(self, total_tokens):
        """The C descriptor (by reference) with total_tokens set. The handle
        keeps this descriptor, and so its tensors, alive."""
        self.c.total_tokens = int(total_tokens)
        return ctypes.byref(self.c)


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace_bytes(desc, total_tokens=0):
    return int(_lib.hp_workspace_bytes(desc.with_tokens(total_tokens)))


def _torch_stream(stream, device):
    """The torch stream object a call runs on (None: the current stream)."""
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _own_workspace(n, device, stream):
    """A workspace the binding allocates for one call. The caching allocator
    hands out blocks per stream, so the block is recorded on the call's
    stream: it is not reused by other work until that stream has passed the
    call, even after the binding drops it."""
    torch = _torch()
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    ws.record_stream(_torch_stream(stream, device))
    return ws


def disjoint_workspace_bytes(desc, total_tokens=0):
    """Workspace bytes of validate_writes and of scatters with disjoint=True."""
    return int(_lib.hp_disjoint_workspace_bytes(desc.with_tokens(total_tokens)))


def _workspace(desc, total_tokens, workspace, stream=None, disjoint=False):
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    n = (disjoint_workspace_bytes if disjoint else workspace_bytes)(desc, total_tokens)
    if n == 0:
        return None, 0
    ws = _own_workspace(n, desc.device, stream)
    desc._ws = ws  # keep alive until the next call on this descriptor
    return ws.data_ptr(), n


def validate(desc, total_tokens, seq_start=None, *, workspace=None, stream=None, result=None):
    """Runs hp_validate; returns (status name, index). Synchronous.

    result: optional 16-byte pinned host tensor to receive the result words
    (the library writes small descriptors' results there directly);
    default: a host struct."""
    p = desc.with_tokens(total_tokens)
    ws, n = _workspace(desc, total_tokens, workspace, stream)
    if result is None:
        res = HpValidateResult()
        res_p = ctypes.byref(res)
    else:
        assert result.numel() * result.element_size() == ctypes.sizeof(HpValidateResult)
        res = HpValidateResult.from_address(result.data_ptr())
        res_p = ctypes.pointer(res)
    code = _lib.hp_validate(p, _ptr(seq_start), ws, n, res_p, _stream(stream, desc.device))
    name = STATUS.get(code, str(code))
    if name == "HP_ERR_HIP":
        raise HpError(code, "hp_validate")
    return name, int(res.index)


def validate_writes(desc, total_tokens, seq_start=None, *, zero_tail=False, workspace=None,
                    stream=None):
    """Runs hp_validate_writes: the descriptor's checks, then whether a
    scatter with these starts (and tail zeroing) writes every slot at most
    once. Returns (status name, index); HP_ERR_WRITE_ALIAS names the smallest
    clashing sequence. Synchronous."""
    p = desc.with_tokens(total_tokens)
    ws, n = _workspace(desc, total_tokens, workspace, stream, disjoint=True)
    res = HpValidateResult()
    code = _lib.hp_validate_writes(p, _ptr(seq_start), HP_FLAG_ZERO_TAIL if zero_tail else 0,
                                   ws, n, ctypes.byref(res), _stream(stream, desc.device))
    name = STATUS.get(code, str(code))
    if name == "HP_ERR_HIP":
        raise HpError(code, "hp_validate_writes")
    return name, int(res.index)


def validate_async(desc, total_tokens, seq_start=None, *, workspace, stream=None):
    """Enqueues hp_validate_async: the verdict stays in the first 16 bytes of
    `workspace` (a device tensor of at least 256 bytes), where moves called
    with gated=True on that workspace read it. Returns at once."""
    p = desc.with_tokens(total_tokens)
    _check(_lib.hp_validate_async(p, _ptr(seq_start), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(stream, desc.device)), "hp_validate_async")


def validate_verdict(desc, total_tokens, workspace):
    """(status name, index) of the verdict hp_validate_async left in
    `workspace` (copied back here; the caller orders this after the check,
    e.g. by synchronizing its stream)."""
    words = workspace[:16].cpu().numpy().tobytes()
    res = HpValidateResult()
    buf = ctypes.create_string_buffer(words, 16)
    _lib.hp_validate_verdict(desc.with_tokens(total_tokens), buf, ctypes.byref(res))
    return STATUS.get(res.code, str(res.code)), int(res.index)


def _flags(checked=False, gated=False, **named):
    f = (HP_FLAG_CHECKED if checked else 0) | (HP_FLAG_GATED if gated else 0)
    for name, on in named.items():
        if on:
            f |= {"streaming": HP_FLAG_STREAM, "zero_tail": HP_FLAG_ZERO_TAIL,
                  "disjoint": HP_FLAG_DISJOINT}[name]
    return f


def gather(desc, out, *, checked=False, streaming=False, workspace=None, stream=None,
           gated=False):
    """out[T, H, D] <- the logical tensor (T = out.shape[0]).

    streaming: hint that no pool page is read twice (slices do not alias), so
    the pool is read with non-temporal loads; the result is the same."""
    T = out.shape[0]
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream)
    flags = _flags(checked, gated, streaming=streaming)
    _check(_lib.hp_gather(p, _ptr(out), ws, n, flags, _stream(stream, desc.device)),
           "hp_gather")
    return out


def gather_static(desc, out, *, checked=False, streaming=False, stream=None):
    """hp_gather_static: the gather with the library's own device workspace
    (no allocation at all; calls on one GPU must not overlap)."""
    p = desc.with_tokens(out.shape[0])
    _check(_lib.hp_gather_static(p, _ptr(out), _flags(checked, False, streaming=streaming),
                                 _stream(stream, desc.device)), "hp_gather_static")
    return out


def scatter(desc, src, seq_start=None, *, zero_tail=False, checked=False, workspace=None,
            stream=None, gated=False, disjoint=False):
    """Writes src[T, H, D] (T = src.shape[0]) into the pool. disjoint: checked,
    and also rejected (HP_ERR_WRITE_ALIAS, nothing written) when two writes
    would land in one slot."""
    T = src.shape[0]
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream, disjoint)
    flags = _flags(checked or disjoint, gated, zero_tail=zero_tail, disjoint=disjoint)
    _check(_lib.hp_scatter(p, _ptr(src), _ptr(seq_start), ws, n, flags,
                           _stream(stream, desc.device)), "hp_scatter")


def gather_dequant(desc, out, *, checked=False, workspace=None, stream=None, gated=False):
    """out[T, H, D] (bfloat16) <- dequantised logical tensor of an int8 pool."""
    T = out.shape[0]
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream)
    _check(_lib.hp_gather_dequant(p, _ptr(out), DTYPE["bf16"], ws, n, _flags(checked, gated),
                                  _stream(stream, desc.device)), "hp_gather_dequant")
    return out


def gather_dequant_q(desc, out, scheme, scales, *, axis=0, block_size=None, zero_points=None,
                     checked=False, workspace=None, stream=None, gated=False):
    """out[T, H, D] (bfloat16) <- dequantised logical tensor of an int8 or
    uint8 pool under a quantization scheme ("per_tensor", "per_channel" with
    axis 1 or 2, "per_block_affine" with axis 0 and block_size = page size).
    scales: float32 device tensor; zero_points: device tensor of the pool's
    element type, or None. desc.scales is not used."""
    T = out.shape[0]
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream)
    q = HpQuant(QUANT_SCHEME[scheme] if isinstance(scheme, str) else int(scheme),
                int(axis), int(desc.c.page_size if block_size is None else block_size),
                _ptr(scales), _ptr(zero_points))
    _check(_lib.hp_gather_dequant_q(p, ctypes.byref(q), _ptr(out), DTYPE["bf16"], ws, n,
                                    _flags(checked, gated),
                                    _stream(stream, desc.device)), "hp_gather_dequant_q")
    return out


def scatter_quant(desc, src, seq_start=None, *, zero_points=None, zero_tail=False,
                  checked=False, workspace=None, stream=None, gated=False, disjoint=False):
    """Quantizes src[T, H, D] (f16, bf16 or f32) into desc's int8 pool
    (symmetric) or uint8 pool (asymmetric, with zero_points: uint8 per slot),
    writing each written slot's scale into desc.scales. disjoint: as in
    scatter."""
    T = src.shape[0]
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream, disjoint)
    flags = _flags(checked or disjoint, gated, zero_tail=zero_tail, disjoint=disjoint)
    _check(_lib.hp_scatter_quant(p, _ptr(src), _dtype_code(src), _ptr(zero_points),
                                 _ptr(seq_start), ws, n, flags, _stream(stream, desc.device)),
           "hp_scatter_quant")


def attention_workspace_bytes(desc, total_tokens, num_q_heads):
    """Workspace bytes of paged_attention (0 for an unsupported shape)."""
    return int(_lib.hp_attention_workspace_bytes(desc.with_tokens(total_tokens), num_q_heads))


def attention_plan(desc, num_q_heads, *, total_tokens, checked=False, streaming=False,
                   workspace=None, stream=None):
    """Runs the attention calls' planning kernels alone into `workspace`
    (allocated through torch when None) and returns it: pass it, with
    planned=True, to paged_attention / paged_attention_q8 calls on the same
    descriptor, query-head count and streaming setting (for instance one per
    layer) and they skip their planning."""
    p = desc.with_tokens(total_tokens)
    n = int(_lib.hp_attention_workspace_bytes(p, num_q_heads))
    if workspace is None:
        workspace = _own_workspace(max(n, 256), desc.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    flags = (HP_FLAG_CHECKED if checked else 0) | (HP_FLAG_STREAM if streaming else 0)
    _check(_lib.hp_attention_plan(p, num_q_heads, _ptr(workspace), ws_bytes, flags,
                                  _stream(stream, desc.device)), "hp_attention_plan")
    return workspace


def _attention(desc, v_pool, v_scales, q, out, total_tokens, scale, checked, streaming,
               workspace, stream, q8, planned=False):
    Hq = q.shape[1]
    p = desc.with_tokens(total_tokens)
    n = int(_lib.hp_attention_workspace_bytes(p, Hq))
    if planned and workspace is None:
        raise ValueError("planned=True needs the workspace attention_plan filled")
    if workspace is None and n:
        workspace = _own_workspace(n, q.device, stream)
        desc._ws = workspace  # keep alive until the next call on this descriptor
    if scale is None:
        scale = 1.0 / float(desc.c.head_dim) ** 0.5
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    flags = ((HP_FLAG_CHECKED if checked else 0) | (HP_FLAG_STREAM if streaming else 0) |
             (HP_FLAG_PLANNED if planned else 0))
    st = _stream(stream, desc.device)
    if q8:
        _check(_lib.hp_paged_attention_q8(p, _ptr(v_pool), _ptr(v_scales), _ptr(q), Hq,
                                          float(scale), _ptr(out), DTYPE["f32"],
                                          _ptr(workspace), ws_bytes, flags, st),
               "hp_paged_attention_q8")
    else:
        _check(_lib.hp_paged_attention(p, _ptr(v_pool), _ptr(q), Hq, float(scale), _ptr(out),
                                       DTYPE["f32"], _ptr(workspace), ws_bytes, flags, st),
               "hp_paged_attention")
    return out


def paged_attention(desc, v_pool, q, out, *, total_tokens, scale=None, checked=False,
                    streaming=False, workspace=None, stream=None, planned=False):
    """out[S, Hq, D] (float32) <- decode attention of q[S, Hq, D] over the K
    cache of `desc` (its page_pool) and the V pool `v_pool`, both read
    through desc's block table. total_tokens: the sum of the token counts.
    scale defaults to 1/sqrt(head_dim). A workspace is allocated through
    torch when none is given. planned: `workspace` holds the plan
    attention_plan wrote for this descriptor and settings."""
    return _attention(desc, v_pool, None, q, out, total_tokens, scale, checked, streaming,
                      workspace, stream, False, planned)


def paged_attention_q8(desc, v_pool, v_scales, q, out, *, total_tokens, scale=None,
                       checked=False, streaming=False, workspace=None, stream=None,
                       planned=False):
    """out[S, Hq, D] (float32) <- decode attention of bf16 q[S, Hq, D] over
    int8 pools with one fp32 scale per slot, each element's value being its
    code times its slot's scale: the K pool and K scales of `desc` (its
    page_pool and scales), the V pool `v_pool` and `v_scales`. Other
    arguments as paged_attention."""
    return _attention(desc, v_pool, v_scales, q, out, total_tokens, scale, checked, streaming,
                      workspace, stream, True, planned)


# ---- batched calls: several pools through the table of one descriptor -------

def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[_ptr(t) for t in tensors])
    return arr


def gather_batch(desc, pools, outs, *, checked=False, streaming=False, workspace=None,
                 stream=None, gated=False):
    """outs[i][T, H, D] <- gather of pools[i] through desc's table (desc's own
    page_pool is ignored). T = outs[0].shape[0]."""
    T = outs[0].shape[0] if len(outs) else 0
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream)
    pa, oa = _ptr_array(pools), _ptr_array(outs)
    flags = _flags(checked, gated, streaming=streaming)
    _check(_lib.hp_gather_batch(p, len(pools), pa, oa, ws, n, flags,
                                _stream(stream, desc.device)), "hp_gather_batch")
    return outs


def scatter_batch(desc, pools, srcs, seq_start=None, *, zero_tail=False, checked=False,
                  workspace=None, stream=None, gated=False, disjoint=False):
    """Writes srcs[i][T, H, D] into pools[i] through desc's table."""
    T = srcs[0].shape[0] if len(srcs) else 0
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream, disjoint)
    pa, sa = _ptr_array(pools), _ptr_array(srcs)
    flags = _flags(checked or disjoint, gated, zero_tail=zero_tail, disjoint=disjoint)
    _check(_lib.hp_scatter_batch(p, len(pools), pa, sa, _ptr(seq_start), ws, n, flags,
                                 _stream(stream, desc.device)), "hp_scatter_batch")


def gather_dequant_batch(desc, pools, scales, outs, *, checked=False, workspace=None,
                         stream=None, gated=False):
    """outs[i] (bf16) <- dequantised gather of int8 pools[i] with scales[i]."""
    T = outs[0].shape[0] if len(outs) else 0
    p = desc.with_tokens(T)
    ws, n = _workspace(desc, T, workspace, stream)
    pa, sa, oa = _ptr_array(pools), _ptr_array(scales), _ptr_array(outs)
    _check(_lib.hp_gather_dequant_batch(p, len(pools), pa, sa, oa, DTYPE["bf16"], ws, n,
                                        _flags(checked, gated),
                                        _stream(stream, desc.device)),
           "hp_gather_dequant_batch")
    return outs


# ---- copy-on-write page copy ----------------------------------------------------

def copy_pages(desc, src_pages, dst_pages, *, checked=False, workspace=None, stream=None):
    """Page dst_pages[i] of desc's pool (and its slot scales) <- page src_pages[i]."""
    n = src_pages.numel()
    if dst_pages.numel() != n:
        raise ValueError("src_pages and dst_pages differ in length")
    p = desc.with_tokens(0)
    ws, wn = _workspace(desc, 0, workspace, stream)
    _check(_lib.hp_copy_pages(p, _ptr(src_pages), _ptr(dst_pages), n, ws, wn,
                              HP_FLAG_CHECKED if checked else 0, _stream(stream, desc.device)),
           "hp_copy_pages")


def copy_pages_batch(desc, pools, scales, src_pages, dst_pages, *, checked=False,
                     workspace=None, stream=None):
    """The same page copies in every pool of `pools` (scales: list or None)."""
    n = src_pages.numel()
    if dst_pages.numel() != n:
        raise ValueError("src_pages and dst_pages differ in length")
    p = desc.with_tokens(0)
    ws, wn = _workspace(desc, 0, workspace, stream)
    pa = _ptr_array(pools)
    sa = _ptr_array(scales) if scales is not None else None
    _check(_lib.hp_copy_pages_batch(p, len(pools), pa, sa, _ptr(src_pages), _ptr(dst_pages), n,
                                    ws, wn, HP_FLAG_CHECKED if checked else 0,
                                    _stream(stream, desc.device)), "hp_copy_pages_batch")
