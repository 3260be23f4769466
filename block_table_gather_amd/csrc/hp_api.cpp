// hp_api.cpp -- the C ABI of include/hp.h: host-side argument checks, launch
// planning and the synchronous validator. Everything that touches data runs
// in the kernels of hp_kernels.hip.
#include "hp.h"
#include "hp_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

namespace {

constexpr uint64_t kValidateBytes = 256;  // workspace head: validator key + sum

// The HIP error behind the calling thread's last HP_ERR_HIP (per thread, so
// concurrent callers do not see each other's errors).
thread_local hipError_t t_last_hip_error = hipSuccess;

hp_status hip_failed(hipError_t e) {
    t_last_hip_error = e;
    return HP_ERR_HIP;
}
constexpr uint64_t kMaxIndex = (1ull << hp::kKeyShift) - 1;

uint32_t elem_bytes_of(uint32_t dtype) {
    switch (dtype) {
    case HP_DTYPE_I8:
    case HP_DTYPE_U8: return 1;
    case HP_DTYPE_F16:
    case HP_DTYPE_BF16: return 2;
    case HP_DTYPE_F32: return 4;
    case HP_DTYPE_F64: return 8;
    default: return 0;
    }
}

bool aligned(const void *p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

bool mul(uint64_t a, uint64_t b, uint64_t *r) { return !__builtin_mul_overflow(a, b, r); }

struct Geometry {
    uint32_t elem_bytes, idx_bytes;
    uint64_t row_bytes, pool_bytes;
};

// Checks shared by every call ([Hurray] Description: rank 3; Logical Shape /
// invariant 6: paged_axis 0; Sharding: no shard descriptor; byte_offset: 0;
// Additional Descriptor Fields: uint32 tables address at most 2^32 pages;
// Alignment: descriptor buffers at least 64-byte aligned).
hp_status check_desc(const hp_desc *d, Geometry *g) {
    if (!d)
        return HP_ERR_NULL;
    if (d->rank != 3)
        return HP_ERR_RANK;
    if (d->paged_axis != 0)
        return HP_ERR_PAGED_AXIS;
    if (d->has_shard)
        return HP_ERR_SHARDED;
    if (d->index_type != HP_INDEX_U32 && d->index_type != HP_INDEX_U64)
        return HP_ERR_INDEX_TYPE;
    g->elem_bytes = elem_bytes_of(d->dtype);
    if (!g->elem_bytes)
        return HP_ERR_DTYPE;
    g->idx_bytes = d->index_type == HP_INDEX_U32 ? 4 : 8;
    if (d->byte_offset != 0)
        return HP_ERR_ARG;
    if (!d->page_size || !d->num_heads || !d->head_dim)
        return HP_ERR_ARG;
    uint64_t hd, tmp;
    if (!mul(d->num_heads, d->head_dim, &hd) || !mul(hd, g->elem_bytes, &g->row_bytes))
        return HP_ERR_ARG;
    // Inner offsets of one work unit are 32-bit; a row must leave room for
    // the dequant output (2 bytes per element) below 2^31.
    if (hd * 2 >= (1ull << 31) || g->row_bytes >= (1ull << 31))
        return HP_ERR_ARG;
    if (!mul(d->num_pages, d->page_size, &tmp) || !mul(tmp, g->row_bytes, &g->pool_bytes))
        return HP_ERR_ARG;
    if (!mul(d->num_block_entries, d->page_size, &tmp))
        return HP_ERR_ARG;
    if (!mul(d->total_tokens, hd * 2 > g->row_bytes ? hd * 2 : g->row_bytes, &tmp))
        return HP_ERR_ARG;
    if (d->num_seqs >= kMaxIndex || d->num_block_entries >= kMaxIndex)
        return HP_ERR_ARG;
    if (d->num_seqs >= (1ull << 32))
        return HP_ERR_ARG;
    if (d->index_type == HP_INDEX_U32 &&
        (d->num_pages > (1ull << 32) || d->num_block_entries > 0xffffffffull))
        return HP_ERR_INDEX_TYPE;
    if (!d->seq_ptr)
        return HP_ERR_NULL;
    if (d->num_block_entries && !d->block_table)
        return HP_ERR_NULL;
    if (d->num_seqs && !d->seq_lens)
        return HP_ERR_NULL;
    if (d->num_pages && !d->page_pool)
        return HP_ERR_NULL;
    if (!aligned(d->page_pool, 64) || !aligned(d->block_table, 64) ||
        !aligned(d->seq_ptr, 64) || !aligned(d->scales, 64) ||
        !aligned(d->seq_lens, g->idx_bytes))
        return HP_ERR_ALIGN;
    return HP_OK;
}

bool overlaps(const void *a, uint64_t an, const void *b, uint64_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return an && bn && x < y + bn && y < x + an;
}

hp_status check_workspace(const void *ws, size_t have, uint64_t need) {
    if (!need)
        return HP_OK;
    if (!ws || have < need)
        return HP_ERR_WORKSPACE;
    if (!aligned(ws, 8))
        return HP_ERR_ALIGN;
    return HP_OK;
}

// Bytes of the plan arrays: needed above kFusedMaxSeqs sequences, and used by
// choice from kPlanMinSeqs on (moves in HP_PLAN_OPS) when the caller's
// workspace holds them.
uint64_t plan_bytes(const hp_desc *d) {
    return d->num_seqs >= hp::kPlanMinSeqs || d->num_seqs > hp::kFusedMaxSeqs
               ? hp::plan_workspace_bytes(d->num_seqs)
               : 0;
}

// Whether a move takes the plan path: always above kFusedMaxSeqs sequences;
// from kPlanMinSeqs on it does when it is one of HP_PLAN_OPS and the
// workspace holds the plan arrays.
bool use_plan(const hp_desc *d, hp::Op op, const void *ws, size_t ws_bytes) {
    if (d->num_seqs > hp::kFusedMaxSeqs)
        return true;
    return hp::plan_preferred(op, d->num_seqs) && ws && ws_bytes >= kValidateBytes + plan_bytes(d);
}

// The validator's two words (smallest failing key, all ones if none; the sum
// of the token counts) as a status and index.
hp_status decode_verdict(const uint64_t words[2], uint64_t total_tokens,
                         hp_validate_result *res) {
    res->code = HP_OK;
    res->reserved = 0;
    res->index = 0;
    if (words[0] != ~0ull) {
        static const hp_status by_rank[] = {HP_OK, HP_ERR_SEQPTR_FIRST, HP_ERR_SEQPTR_LAST,
                                            HP_ERR_SEQPTR_ORDER, HP_ERR_PAGE_RANGE,
                                            HP_ERR_SEQ_LEN};
        const uint64_t rank = words[0] >> hp::kKeyShift;
        res->code = rank >= 1 && rank <= 5 ? by_rank[rank] : HP_ERR_HIP;
        res->index = words[0] & kMaxIndex;
    } else if (words[1] != total_tokens) {
        res->code = HP_ERR_TOTAL_TOKENS;
    }
    return (hp_status)res->code;
}

hp::ValidateJob validate_job(const hp_desc *d, const void *seq_start, void *ws) {
    hp::ValidateJob j;
    j.idx64 = d->index_type == HP_INDEX_U64;
    j.num_pages = d->num_pages;
    j.page_size = d->page_size;
    j.num_seqs = d->num_seqs;
    j.num_block_entries = d->num_block_entries;
    j.block_table = d->block_table;
    j.seq_ptr = d->seq_ptr;
    j.seq_lens = d->seq_lens;
    j.seq_start = seq_start;
    j.workspace = ws;
    j.result = nullptr;
    return j;
}

hp_status run_validate(const hp_desc *d, const void *seq_start, void *ws,
                       hp_validate_result *res, hipStream_t stream) {
    hp::ValidateJob j = validate_job(d, seq_start, ws);
    // The two result words land in the caller's result struct (16 bytes, like
    // them) and are decoded in place after the wait. When the struct is
    // pinned host memory the GPU can reach, a small descriptor's check writes
    // them there itself; otherwise they are copied from the workspace.
    static_assert(sizeof(hp_validate_result) == 2 * sizeof(uint64_t), "result layout");
    j.result = nullptr;
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, res) == hipSuccess && attr.type == hipMemoryTypeHost &&
        attr.devicePointer)
        j.result = attr.devicePointer;
    (void)hipGetLastError();  // an unregistered pointer leaves an error behind
    hipError_t e = hp::launch_validate(j, stream);
    if (e != hipSuccess)
        return hip_failed(e);
    if (!hp::validate_writes_result(j) &&
        (e = hipMemcpyAsync(res, ws, sizeof(hp_validate_result), hipMemcpyDeviceToHost,
                            stream)) != hipSuccess)
        return hip_failed(e);
    if ((e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_failed(e);
    uint64_t host[2];
    memcpy(host, res, sizeof host);
    return decode_verdict(host, d->total_tokens, res);
}

// Bytes hp_validate_writes needs: the validator's words, the answer and the
// two slot bitmaps, and never less than a move's workspace.
uint64_t disjoint_bytes(const hp_desc *d) {
    const uint64_t a = hp::disjoint_workspace_bytes(d->num_pages, d->page_size);
    const uint64_t b = kValidateBytes + plan_bytes(d);
    return a > b ? a : b;
}

// Write-disjointness on a validated descriptor: HP_ERR_WRITE_ALIAS with the
// smallest clashing sequence, or HP_OK. Synchronous.
hp_status run_disjoint(const hp_desc *d, const void *seq_start, bool zero_tail, void *ws,
                       hp_validate_result *res, hipStream_t stream) {
    hp::DisjointJob j;
    j.idx64 = d->index_type == HP_INDEX_U64;
    j.zero_tail = zero_tail;
    j.num_pages = d->num_pages;
    j.page_size = d->page_size;
    j.num_seqs = d->num_seqs;
    j.block_table = d->block_table;
    j.seq_ptr = d->seq_ptr;
    j.seq_lens = d->seq_lens;
    j.seq_start = seq_start;
    j.workspace = ws;
    hipError_t e = hp::launch_disjoint(j, stream);
    if (e != hipSuccess)
        return hip_failed(e);
    uint64_t answer = 0;
    if ((e = hipMemcpyAsync(&answer, static_cast<unsigned char *>(ws) + hp::kDisjointAnswer,
                            sizeof answer, hipMemcpyDeviceToHost, stream)) != hipSuccess)
        return hip_failed(e);
    if ((e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_failed(e);
    res->code = HP_OK;
    res->reserved = 0;
    res->index = 0;
    if (answer != ~0ull) {
        res->code = HP_ERR_WRITE_ALIAS;
        res->index = answer;
    }
    return (hp_status)res->code;
}

// Largest divisor of P whose run of rows fits the target unit size (at least
// 1, at most `cap`).
uint32_t rows_per_unit(uint32_t P, uint64_t row_bytes, uint64_t unit_bytes, uint32_t cap) {
    uint64_t want = unit_bytes / (row_bytes ? row_bytes : 1);
    if (want < 1)
        want = 1;
    if (want > cap)
        want = cap;
    if (want > P)
        want = P;
    for (uint32_t r = (uint32_t)want; r > 1; --r)
        if (P % r == 0)
            return r;
    return 1;
}

// The pools and logical tensors one call moves: `count` of each (a single
// call passes one), plus the per-slot scales of a dequant.
struct Members {
    uint32_t count;
    void *const *pools;
    void *const *rows;
    const float *const *scales;
};

// Widest vector (in source bytes) that divides a row and keeps every pool
// access, and every logical-tensor access (out_scale bytes per source byte),
// aligned.
uint32_t widest_vec(uint64_t row_bytes, const Members &m, uint32_t maxv, uint32_t out_scale) {
    for (uint32_t v = maxv; v > 1; v >>= 1) {
        bool ok = row_bytes % v == 0;
        for (uint32_t i = 0; ok && i < m.count; ++i)
            ok = aligned(m.pools[i], v) && aligned(m.rows[i], (uint64_t)v * out_scale);
        if (ok)
            return v;
    }
    return 1;
}

// A dequant scheme other than the per-slot, symmetric, int8 fast path.
struct QuantSpec {
    bool ext;            // use the general dequant kernel
    uint32_t mode;       // 0 per-slot, 1 per-tensor, 2 per-head, 3 per-head_dim
    bool is_unsigned;
    const float *scales;
    const void *zero_points;
};

hp_status launch(const hp_desc *d, const Geometry &g, hp::Op op, const Members &m,
                 const void *seq_start, uint32_t flags, void *ws, size_t ws_bytes,
                 hipStream_t stream, const QuantSpec *q = nullptr) {
    const bool zero_tail = (flags & HP_FLAG_ZERO_TAIL) != 0;
    hp::CopyJob j = {};
    j.op = op;
    j.idx64 = d->index_type == HP_INDEX_U64;
    j.zero_tail = zero_tail;
    j.elem_bytes = g.elem_bytes;
    j.page_size = d->page_size;
    j.num_seqs = d->num_seqs;
    j.total_tokens = d->total_tokens;
    j.row_bytes = g.row_bytes;
    j.out_row_bytes = op == hp::Op::Dequant ? g.row_bytes * 2 : g.row_bytes;
    const uint64_t rmax = j.out_row_bytes > j.row_bytes ? j.out_row_bytes : j.row_bytes;
    // Per-move launch shape (measured on MI355X): target unit size, units per
    // workgroup, and whether the source is streamed with non-temporal loads.
    j.plan = use_plan(d, op, ws, ws_bytes);
    uint64_t unit_bytes;
    switch (op) {
    case hp::Op::Gather:
        // the fused scan's per-sequence reads are amortised over larger units
        unit_bytes = HP_GATHER_UNIT_BYTES;
        if (!j.plan && d->num_seqs * HP_GATHER_UNIT_BYTES_PER_SEQ > unit_bytes)
            unit_bytes = d->num_seqs * HP_GATHER_UNIT_BYTES_PER_SEQ;
        j.units_per_group = HP_GATHER_UNITS_PER_GROUP;
        j.load_nt = (flags & HP_FLAG_STREAM) != 0;
        break;
    case hp::Op::Scatter:
        // bytes moved by the whole call: count * T * R read and written
        if ((uint64_t)m.count * d->total_tokens * g.row_bytes >= HP_SCATTER_STREAM_BYTES / 2) {
            unit_bytes = HP_SCATTER_STREAM_UNIT_BYTES;
            j.units_per_group = 1;
            j.load_nt = true;
        } else {
            unit_bytes = HP_SCATTER_UNIT_BYTES;
            j.units_per_group = HP_SCATTER_UNITS_PER_GROUP;
            j.load_nt = false;
        }
        break;
    default:
        unit_bytes = HP_DEQUANT_UNIT_BYTES;
        j.units_per_group = HP_DEQUANT_UNITS_PER_GROUP;
        j.load_nt = false;
        break;
    }
    j.rows_per_unit =
        rows_per_unit(d->page_size, rmax, unit_bytes, op == hp::Op::Dequant ? 64 : 0xffffffffu);
    const uint64_t rpc = j.rows_per_unit;
    const uint64_t upp = d->page_size / rpc;
    // Upper bound on the number of units, from host-known T and S only.
    if (op == hp::Op::Scatter)
        j.unit_bound = d->total_tokens / rpc + d->num_seqs * (2 + (zero_tail ? upp : 0));
    else
        j.unit_bound = d->total_tokens / rpc + d->num_seqs;
    if (j.unit_bound >= (1ull << 32) - hp::kMaxUnitsPerGroup)
        return HP_ERR_ARG;
    j.block_table = d->block_table;
    j.seq_ptr = d->seq_ptr;
    j.seq_lens = d->seq_lens;
    j.seq_start = seq_start;
    j.count = m.count;
    j.pools = m.pools;
    j.rows = m.rows;
    j.scales = m.scales;
    j.workspace = ws ? static_cast<unsigned char *>(ws) + kValidateBytes : nullptr;
    j.vec_bytes = op == hp::Op::Dequant ? widest_vec(g.row_bytes, m, 8, 2)
                                        : widest_vec(g.row_bytes, m, 16, 1);
    if (flags & HP_FLAG_GATED) {
        j.gate = static_cast<const unsigned long long *>(ws);
        j.gate_tokens = d->total_tokens;
    }
    if (q) {
        j.quant_ext = q->ext;
        j.quant_mode = q->mode;
        j.quant_unsigned = q->is_unsigned;
        j.quant_scales = q->scales;
        j.zero_points = q->zero_points;
        j.head_dim = d->head_dim;
        j.quant_channels = q->mode == 2 ? d->num_heads : q->mode == 3 ? d->head_dim : 0;
    }
    const hipError_t e = hp::launch_copy(j, stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

// Common front half of gather / scatter / dequant, after the descriptor and
// the call's own buffers were checked: flags, workspace, optional
// validation. *done is set when nothing is left to do.
hp_status prologue(const hp_desc *d, const Geometry &g, uint32_t flags, uint32_t allowed,
                   const void *seq_start, void *ws, size_t ws_bytes, hipStream_t stream,
                   bool *done) {
    *done = false;
    if (flags & ~(allowed | HP_FLAG_GATED))
        return HP_ERR_ARG;
    const bool checked = flags & HP_FLAG_CHECKED;
    const bool gated = flags & HP_FLAG_GATED;
    const bool disjoint = flags & HP_FLAG_DISJOINT;
    if (checked && gated)
        return HP_ERR_ARG;  // one of the two ways of validating
    if (disjoint && !checked)
        return HP_ERR_ARG;  // the clash check runs after the synchronous validation
    if (!aligned(seq_start, g.idx_bytes))
        return HP_ERR_ALIGN;
    const bool fused = d->num_seqs <= hp::kFusedMaxSeqs;
    uint64_t need = !fused ? kValidateBytes + plan_bytes(d)
                           : ((checked || gated) ? kValidateBytes : 0);
    if (disjoint)
        need = disjoint_bytes(d);
    hp_status st = check_workspace(ws, ws_bytes, need);
    if (st != HP_OK)
        return st;
    if (checked) {
        hp_validate_result r;
        st = run_validate(d, seq_start, ws, &r, stream);
        if (st != HP_OK)
            return st;
        // the bitmaps share the plan's part of the workspace: the host has
        // waited for the check before the move is enqueued
        if (disjoint && (st = run_disjoint(d, seq_start, flags & HP_FLAG_ZERO_TAIL, ws, &r,
                                           stream)) != HP_OK)
            return st;
    }
    *done = d->num_seqs == 0 || d->total_tokens == 0;
    return HP_OK;
}

// Checks shared by the batched calls: the descriptor (with pools[0] standing
// in for its page_pool and scales[0] for its scales), every member pointer,
// and that no written buffer overlaps another buffer of the call.
hp_status check_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                      void *const *rows, const float *const *scales, bool rows_written,
                      bool need_scales, hp_desc *local, Geometry *g) {
    if (!desc || !pools || !rows || (need_scales && !scales))
        return HP_ERR_NULL;
    *local = *desc;
    local->page_pool = pools[0];
    local->scales = need_scales ? scales[0] : nullptr;
    hp_status st = check_desc(local, g);
    if (st != HP_OK)
        return st;
    const uint64_t rows_bytes =
        local->total_tokens * g->row_bytes * (need_scales ? 2 : 1);  // dequant writes bf16
    const uint32_t row_align = need_scales ? 2 : g->elem_bytes;
    const uint64_t scale_bytes = local->num_pages * local->page_size * 4;
    for (uint32_t i = 0; i < count; ++i) {
        if ((local->num_pages && !pools[i]) || (local->total_tokens && !rows[i]) ||
            (need_scales && !scales[i]))
            return HP_ERR_NULL;
        if (!aligned(pools[i], 64) || !aligned(rows[i], row_align) ||
            (need_scales && !aligned(scales[i], 64)))
            return HP_ERR_ALIGN;
    }
    for (uint32_t i = 0; i < count; ++i) {
        for (uint32_t k = 0; k < count; ++k) {
            // a logical tensor never overlaps a pool or scales; written buffers
            // of different members never overlap each other
            if (overlaps(rows[i], rows_bytes, pools[k], g->pool_bytes) ||
                (need_scales && overlaps(rows[i], rows_bytes, scales[k], scale_bytes)))
                return HP_ERR_ARG;
            if (i != k && rows_written && overlaps(rows[i], rows_bytes, rows[k], rows_bytes))
                return HP_ERR_ARG;
            if (i != k && !rows_written && overlaps(pools[i], g->pool_bytes, pools[k], g->pool_bytes))
                return HP_ERR_ARG;
        }
    }
    return HP_OK;
}

// Shared by hp_copy_pages and hp_copy_pages_batch: every pool of the call
// gets the same page copies.
hp_status copy_pages_common(const hp_desc *desc, uint32_t num_pools, void *const *pools,
                            float *const *scales, const void *src_pages, const void *dst_pages,
                            uint64_t copies, void *ws, size_t ws_bytes, uint32_t flags,
                            hipStream_t stream) {
    if (!desc || !pools)
        return HP_ERR_NULL;
    if (num_pools == 0)
        return HP_OK;
    hp_desc d = *desc;
    d.page_pool = pools[0];
    d.scales = scales ? scales[0] : nullptr;
    Geometry g;
    hp_status st = check_desc(&d, &g);
    if (st != HP_OK)
        return st;
    if (flags & ~(uint32_t)HP_FLAG_CHECKED)
        return HP_ERR_ARG;
    const uint64_t page_bytes = (uint64_t)d.page_size * g.row_bytes;
    if (page_bytes >= (1ull << 32))
        return HP_ERR_ARG;
    for (uint32_t i = 0; i < num_pools; ++i) {
        if (d.num_pages && !pools[i])
            return HP_ERR_NULL;
        if (!aligned(pools[i], 64) || (scales && !aligned(scales[i], 64)))
            return HP_ERR_ALIGN;
        for (uint32_t k = 0; k < i; ++k)
            if (overlaps(pools[i], g.pool_bytes, pools[k], g.pool_bytes))
                return HP_ERR_ARG;
    }
    if (copies == 0)
        return HP_OK;
    if (!src_pages || !dst_pages)
        return HP_ERR_NULL;
    if (!aligned(src_pages, g.idx_bytes) || !aligned(dst_pages, g.idx_bytes))
        return HP_ERR_ALIGN;
    const uint64_t chunks = (page_bytes + hp::kPageChunkBytes - 1) / hp::kPageChunkBytes;
    if (copies >= kMaxIndex || copies * chunks >= (1ull << 31))
        return HP_ERR_ARG;
    if (flags & HP_FLAG_CHECKED) {
        if ((st = check_workspace(ws, ws_bytes, kValidateBytes)) != HP_OK)
            return st;
        hp::PageCheckJob c;
        c.idx64 = d.index_type == HP_INDEX_U64;
        c.copies = copies;
        c.num_pages = d.num_pages;
        c.src_pages = src_pages;
        c.dst_pages = dst_pages;
        c.workspace = ws;
        hipError_t e = hp::launch_check_pages(c, stream);
        uint64_t key = 0;
        if (e == hipSuccess)
            e = hipMemcpyAsync(&key, ws, sizeof key, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess)
            e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return hip_failed(e);
        if (key != ~0ull)
            return HP_ERR_PAGE_RANGE;
    }
    hp::PageCopyJob j;
    j.idx64 = d.index_type == HP_INDEX_U64;
    j.vec_bytes = 16;
    while (j.vec_bytes > 1 && page_bytes % j.vec_bytes)
        j.vec_bytes >>= 1;
    j.page_size = d.page_size;
    j.page_bytes = page_bytes;
    j.copies = copies;
    j.src_pages = src_pages;
    j.dst_pages = dst_pages;
    j.count = num_pools;
    j.pools = pools;
    j.scales = scales;
    const hipError_t e = hp::launch_copy_pages(j, stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

// ---- the allocation-free gather ------------------------------------------------
//
// hp_gather_static keeps its workspace in this file-scope device array: the
// validator's words (HP_FLAG_CHECKED) and the plan arrays of calls over many
// sequences. Each GPU the library runs on holds its own copy until the
// process ends. Host code never passes the array's name to a kernel or a
// copy: it stands for a host-side shadow there. The device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr uint64_t kStaticMaxSeqs = 1u << 18;
constexpr uint64_t kStaticScratchBytes = 256 + 0x300800;  // validator + plan at kStaticMaxSeqs
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The current device's copy of `scratch` (its device address), or null with
// the HIP error in *e.
void *device_scratch(hipError_t *e) {
    int dev = 0;
    if ((*e = hipGetDevice(&dev)) != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *e = hipErrorInvalidDevice;
        return nullptr;
    }
    DeviceScratch &d = g_scratch[dev];
    std::call_once(d.once, [&d] {
        void *ptr = nullptr;
        d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        d.ptr = d.err == hipSuccess ? ptr : nullptr;
    });
    *e = d.err;
    return d.ptr;
}

} // namespace

extern "C" {

size_t hp_workspace_bytes(const hp_desc *desc) {
    Geometry g;
    if (check_desc(desc, &g) != HP_OK)
        return 0;
    return (size_t)(kValidateBytes + plan_bytes(desc));
}

size_t hp_disjoint_workspace_bytes(const hp_desc *desc) {
    Geometry g;
    if (check_desc(desc, &g) != HP_OK)
        return 0;
    return (size_t)disjoint_bytes(desc);
}

hp_status hp_validate_writes(const hp_desc *desc, const void *seq_start, uint32_t flags,
                             void *workspace, size_t workspace_bytes,
                             hp_validate_result *result, void *stream) {
    hp_validate_result local;
    hp_validate_result *res = result ? result : &local;
    res->code = HP_OK;
    res->reserved = 0;
    res->index = 0;
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st == HP_OK && (flags & ~(uint32_t)HP_FLAG_ZERO_TAIL))
        st = HP_ERR_ARG;
    if (st == HP_OK && !aligned(seq_start, g.idx_bytes))
        st = HP_ERR_ALIGN;
    if (st == HP_OK)
        st = check_workspace(workspace, workspace_bytes, disjoint_bytes(desc));
    if (st != HP_OK) {
        res->code = st;
        return st;
    }
    if ((st = run_validate(desc, seq_start, workspace, res, (hipStream_t)stream)) != HP_OK)
        return st;
    return run_disjoint(desc, seq_start, flags & HP_FLAG_ZERO_TAIL, workspace, res,
                        (hipStream_t)stream);
}

hp_status hp_validate(const hp_desc *desc, const void *seq_start, void *workspace,
                      size_t workspace_bytes, hp_validate_result *result, void *stream) {
    hp_validate_result local;
    hp_validate_result *res = result ? result : &local;
    res->code = HP_OK;
    res->reserved = 0;
    res->index = 0;
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st == HP_OK && !aligned(seq_start, g.idx_bytes))
        st = HP_ERR_ALIGN;
    if (st == HP_OK)
        st = check_workspace(workspace, workspace_bytes, kValidateBytes);
    if (st != HP_OK) {
        res->code = st;
        return st;
    }
    return run_validate(desc, seq_start, workspace, res, (hipStream_t)stream);
}

hp_status hp_validate_async(const hp_desc *desc, const void *seq_start, void *workspace,
                            size_t workspace_bytes, void *stream) {
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (!aligned(seq_start, g.idx_bytes))
        return HP_ERR_ALIGN;
    if ((st = check_workspace(workspace, workspace_bytes, kValidateBytes)) != HP_OK)
        return st;
    const hipError_t e =
        hp::launch_validate(validate_job(desc, seq_start, workspace), (hipStream_t)stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

hp_status hp_validate_verdict(const hp_desc *desc, const void *words,
                              hp_validate_result *result) {
    if (!desc || !words || !result)
        return HP_ERR_NULL;
    uint64_t w[2];
    memcpy(w, words, sizeof w);
    return decode_verdict(w, desc->total_tokens, result);
}

hp_status hp_gather(const hp_desc *desc, void *out, void *workspace, size_t workspace_bytes,
                    uint32_t flags, void *stream) {
    Geometry g;
    bool done;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (desc->total_tokens && !out)
        return HP_ERR_NULL;
    if (!aligned(out, g.elem_bytes))
        return HP_ERR_ALIGN;
    if (overlaps(out, desc->total_tokens * g.row_bytes, desc->page_pool, g.pool_bytes))
        return HP_ERR_ARG;
    st = prologue(desc, g, flags, HP_FLAG_CHECKED | HP_FLAG_STREAM, nullptr, workspace,
                  workspace_bytes, (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    void *pool = desc->page_pool;
    const Members m = {1, &pool, &out, nullptr};
    return launch(desc, g, hp::Op::Gather, m, nullptr, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

hp_status hp_gather_static(const hp_desc *desc, void *out, uint32_t flags, void *stream) {
    static_assert(kValidateBytes + 8 * kStaticMaxSeqs + 4 * kStaticMaxSeqs +
                          16 * ((kStaticMaxSeqs + hp::kPlanChunk - 1) / hp::kPlanChunk) <=
                      kStaticScratchBytes,
                  "the static workspace holds the plan of kStaticMaxSeqs sequences");
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (flags & ~(uint32_t)(HP_FLAG_CHECKED | HP_FLAG_STREAM))
        return HP_ERR_ARG;  // a gated call needs a verdict only the caller's workspace holds
    if (desc->num_seqs > kStaticMaxSeqs ||
        kValidateBytes + plan_bytes(desc) > kStaticScratchBytes)
        return HP_ERR_WORKSPACE;
    if (desc->total_tokens && !out)
        return HP_ERR_NULL;
    if (!aligned(out, g.elem_bytes))
        return HP_ERR_ALIGN;
    if (overlaps(out, desc->total_tokens * g.row_bytes, desc->page_pool, g.pool_bytes))
        return HP_ERR_ARG;
    if (desc->num_seqs == 0 || desc->total_tokens == 0)
        return HP_OK;  // nothing to move: the device is not touched
    hipError_t e;
    void *ws = device_scratch(&e);
    if (!ws)
        return hip_failed(e);
    return hp_gather(desc, out, ws, kStaticScratchBytes, flags, stream);
}

hp_status hp_scatter(const hp_desc *desc, const void *src, const void *seq_start,
                     void *workspace, size_t workspace_bytes, uint32_t flags, void *stream) {
    Geometry g;
    bool done;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (desc->total_tokens && !src)
        return HP_ERR_NULL;
    if (!aligned(src, g.elem_bytes))
        return HP_ERR_ALIGN;
    if (overlaps(src, desc->total_tokens * g.row_bytes, desc->page_pool, g.pool_bytes))
        return HP_ERR_ARG;
    st = prologue(desc, g, flags, HP_FLAG_CHECKED | HP_FLAG_ZERO_TAIL | HP_FLAG_DISJOINT,
                  seq_start, workspace, workspace_bytes, (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    void *pool = desc->page_pool;
    void *rows = const_cast<void *>(src);  // read, never written
    const Members m = {1, &pool, &rows, nullptr};
    return launch(desc, g, hp::Op::Scatter, m, seq_start, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

hp_status hp_scatter_quant(const hp_desc *desc, const void *src, uint32_t src_dtype,
                           void *zero_points, const void *seq_start, void *workspace,
                           size_t workspace_bytes, uint32_t flags, void *stream) {
    Geometry g;
    bool done;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    const bool asym = desc->dtype == HP_DTYPE_U8;
    if (desc->dtype != HP_DTYPE_I8 && !asym)
        return HP_ERR_DTYPE;
    uint32_t src_code, src_bytes;
    switch (src_dtype) {
    case HP_DTYPE_F16: src_code = 0; src_bytes = 2; break;
    case HP_DTYPE_BF16: src_code = 1; src_bytes = 2; break;
    case HP_DTYPE_F32: src_code = 2; src_bytes = 4; break;
    default: return HP_ERR_DTYPE;
    }
    if (!asym && zero_points)
        return HP_ERR_ARG;  // int8 pools are symmetric: no zero points
    if (desc->num_pages && (!desc->scales || (asym && !zero_points)))
        return HP_ERR_NULL;
    if (desc->total_tokens && !src)
        return HP_ERR_NULL;
    if (!aligned(src, src_bytes) || !aligned(zero_points, 64))
        return HP_ERR_ALIGN;
    const uint64_t n = g.row_bytes;  // one byte per value
    const uint64_t src_row = n * src_bytes, slots = desc->num_pages * desc->page_size;
    const void *written[3] = {desc->page_pool, desc->scales, zero_points};
    const uint64_t wbytes[3] = {g.pool_bytes, 4 * slots, asym ? slots : 0};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(src, desc->total_tokens * src_row, written[i], wbytes[i]))
            return HP_ERR_ARG;
        for (int k = i + 1; k < 3; ++k)
            if (overlaps(written[i], wbytes[i], written[k], wbytes[k]))
                return HP_ERR_ARG;
    }
    st = prologue(desc, g, flags, HP_FLAG_CHECKED | HP_FLAG_ZERO_TAIL | HP_FLAG_DISJOINT,
                  seq_start, workspace, workspace_bytes, (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    const bool zero_tail = (flags & HP_FLAG_ZERO_TAIL) != 0;
    void *pool = desc->page_pool;
    void *rows = const_cast<void *>(src);  // read, never written
    hp::CopyJob j = {};
    j.op = hp::Op::ScatterQuant;
    j.idx64 = desc->index_type == HP_INDEX_U64;
    j.zero_tail = zero_tail;
    j.elem_bytes = 1;
    j.page_size = desc->page_size;
    j.num_seqs = desc->num_seqs;
    j.total_tokens = desc->total_tokens;
    j.row_bytes = n;
    j.out_row_bytes = src_row;
    // 8 values per vector when rows and the source allow 16-byte (or 2 x 16)
    // loads and 8-byte code stores; single values otherwise
    j.vec_bytes = (n % 8 == 0 && aligned(src, 16)) ? 16 : 1;
    // With 16-byte vectors and few sequences a unit is one slot, quantized by
    // a one-wave workgroup; otherwise a unit is a run of consecutive slots of
    // a page and each wave of the workgroup quantizes whole rows of it.
    j.qs_wave_groups = j.vec_bytes == 16 && desc->num_seqs <= hp::kQuantWaveMaxSeqs;
    j.rows_per_unit = j.qs_wave_groups
                          ? 1
                          : rows_per_unit(desc->page_size, 1, HP_QUANT_UNIT_ROWS, 0xffffffffu);
    j.units_per_group = HP_QUANT_UNITS_PER_GROUP;
    const uint64_t upp = desc->page_size / j.rows_per_unit;
    j.unit_bound = desc->total_tokens / j.rows_per_unit +
                   desc->num_seqs * (2 + (zero_tail ? upp : 0));
    if (j.unit_bound >= (1ull << 32) - hp::kMaxUnitsPerGroup)
        return HP_ERR_ARG;
    j.block_table = desc->block_table;
    j.seq_ptr = desc->seq_ptr;
    j.seq_lens = desc->seq_lens;
    j.seq_start = seq_start;
    j.count = 1;
    j.pools = &pool;
    j.rows = &rows;
    j.workspace = workspace ? static_cast<unsigned char *>(workspace) + kValidateBytes : nullptr;
    j.plan = use_plan(desc, hp::Op::ScatterQuant, workspace, workspace_bytes);
    j.qs_src = src_code;
    j.qs_asym = asym;
    j.qs_scales = const_cast<float *>(desc->scales);
    j.qs_zero_points = static_cast<uint8_t *>(zero_points);
    if (flags & HP_FLAG_GATED) {
        j.gate = static_cast<const unsigned long long *>(workspace);
        j.gate_tokens = desc->total_tokens;
    }
    const hipError_t e = hp::launch_copy(j, (hipStream_t)stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

hp_status hp_gather_dequant(const hp_desc *desc, void *out, uint32_t out_dtype, void *workspace,
                            size_t workspace_bytes, uint32_t flags, void *stream) {
    Geometry g;
    bool done;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (desc->dtype != HP_DTYPE_I8 || out_dtype != HP_DTYPE_BF16)
        return HP_ERR_DTYPE;
    if (!desc->scales || (desc->total_tokens && !out))
        return HP_ERR_NULL;
    if (!aligned(out, 2))
        return HP_ERR_ALIGN;
    const uint64_t out_bytes = desc->total_tokens * g.row_bytes * 2;
    if (overlaps(out, out_bytes, desc->page_pool, g.pool_bytes) ||
        overlaps(out, out_bytes, desc->scales, desc->num_pages * desc->page_size * 4))
        return HP_ERR_ARG;
    st = prologue(desc, g, flags, HP_FLAG_CHECKED, nullptr, workspace, workspace_bytes,
                  (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    void *pool = desc->page_pool;
    const float *scales = desc->scales;
    const Members m = {1, &pool, &out, &scales};
    return launch(desc, g, hp::Op::Dequant, m, nullptr, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

// ---- batched calls: several pools through one shared table --------------------

hp_status hp_gather_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                          void *const *outs, void *workspace, size_t workspace_bytes,
                          uint32_t flags, void *stream) {
    if (!desc)
        return HP_ERR_NULL;
    if (count == 0)
        return HP_OK;
    hp_desc d;
    Geometry g;
    bool done;
    hp_status st = check_batch(desc, count, pools, outs, nullptr, true, false, &d, &g);
    if (st != HP_OK)
        return st;
    st = prologue(&d, g, flags, HP_FLAG_CHECKED | HP_FLAG_STREAM, nullptr, workspace,
                  workspace_bytes, (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    const Members m = {count, pools, outs, nullptr};
    return launch(&d, g, hp::Op::Gather, m, nullptr, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

hp_status hp_scatter_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                           const void *const *srcs, const void *seq_start, void *workspace,
                           size_t workspace_bytes, uint32_t flags, void *stream) {
    if (!desc)
        return HP_ERR_NULL;
    if (count == 0)
        return HP_OK;
    hp_desc d;
    Geometry g;
    bool done;
    void *const *rows = const_cast<void *const *>(srcs);  // read, never written
    hp_status st = check_batch(desc, count, pools, rows, nullptr, false, false, &d, &g);
    if (st != HP_OK)
        return st;
    st = prologue(&d, g, flags, HP_FLAG_CHECKED | HP_FLAG_ZERO_TAIL | HP_FLAG_DISJOINT,
                  seq_start, workspace, workspace_bytes, (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    const Members m = {count, pools, rows, nullptr};
    return launch(&d, g, hp::Op::Scatter, m, seq_start, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

hp_status hp_gather_dequant_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                                  const float *const *scales, void *const *outs,
                                  uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                                  uint32_t flags, void *stream) {
    if (!desc)
        return HP_ERR_NULL;
    if (count == 0)
        return HP_OK;
    hp_desc d;
    Geometry g;
    bool done;
    hp_status st = check_batch(desc, count, pools, outs, scales, true, true, &d, &g);
    if (st != HP_OK)
        return st;
    if (d.dtype != HP_DTYPE_I8 || out_dtype != HP_DTYPE_BF16)
        return HP_ERR_DTYPE;
    st = prologue(&d, g, flags, HP_FLAG_CHECKED, nullptr, workspace, workspace_bytes,
                  (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    const Members m = {count, pools, outs, scales};
    return launch(&d, g, hp::Op::Dequant, m, nullptr, flags, workspace, workspace_bytes,
                  (hipStream_t)stream);
}

hp_status hp_gather_dequant_q(const hp_desc *desc, const hp_quant *quant, void *out,
                              uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                              uint32_t flags, void *stream) {
    Geometry g;
    bool done;
    if (!desc || !quant)
        return HP_ERR_NULL;
    hp_desc d = *desc;
    d.scales = quant->scales;  // the scheme's scales replace the descriptor's
    hp_status st = check_desc(&d, &g);
    if (st != HP_OK)
        return st;
    if ((d.dtype != HP_DTYPE_I8 && d.dtype != HP_DTYPE_U8) || out_dtype != HP_DTYPE_BF16)
        return HP_ERR_DTYPE;
    uint32_t mode;
    switch (quant->scheme) {
    case HP_QUANT_PER_TENSOR: mode = 1; break;
    case HP_QUANT_PER_CHANNEL:
        if (quant->axis != 1 && quant->axis != 2)
            return HP_ERR_QUANT;
        mode = quant->axis == 1 ? 2 : 3;
        break;
    case HP_QUANT_PER_BLOCK_AFFINE:
        if (quant->axis != 0 || quant->block_size != d.page_size)
            return HP_ERR_QUANT;
        mode = 0;
        break;
    default: return HP_ERR_QUANT;
    }
    if (!quant->scales || (d.total_tokens && !out))
        return HP_ERR_NULL;
    if (!aligned(quant->scales, 64) || !aligned(quant->zero_points, 64) || !aligned(out, 2))
        return HP_ERR_ALIGN;
    const uint64_t out_bytes = d.total_tokens * g.row_bytes * 2;
    const uint64_t n_params = mode == 0 ? d.num_pages * d.page_size
                              : mode == 1 ? 1 : mode == 2 ? d.num_heads : d.head_dim;
    if (overlaps(out, out_bytes, d.page_pool, g.pool_bytes) ||
        overlaps(out, out_bytes, quant->scales, n_params * 4) ||
        overlaps(out, out_bytes, quant->zero_points, n_params))
        return HP_ERR_ARG;
    st = prologue(&d, g, flags, HP_FLAG_CHECKED, nullptr, workspace, workspace_bytes,
                  (hipStream_t)stream, &done);
    if (st != HP_OK || done)
        return st;
    void *pool = d.page_pool;
    const float *scales = quant->scales;
    const Members m = {1, &pool, &out, &scales};
    QuantSpec q;
    q.ext = !(mode == 0 && !quant->zero_points && d.dtype == HP_DTYPE_I8);
    q.mode = mode;
    q.is_unsigned = d.dtype == HP_DTYPE_U8;
    q.scales = quant->scales;
    q.zero_points = quant->zero_points;
    return launch(&d, g, hp::Op::Dequant, m, nullptr, flags, workspace, workspace_bytes,
                  (hipStream_t)stream, &q);
}

// Shape checks of the attention calls beyond the descriptor's own: the pool
// type is f16 or bf16 (hp_paged_attention) or int8 (hp_paged_attention_q8).
static hp_status check_attention(const hp_desc *d, uint32_t num_q_heads, bool q8) {
    if (q8 ? d->dtype != HP_DTYPE_I8 : d->dtype != HP_DTYPE_F16 && d->dtype != HP_DTYPE_BF16)
        return HP_ERR_DTYPE;
    const uint32_t D = d->head_dim;
    if (D != 8 && D != 16 && D != 32 && D != 64 && D != 128 && D != 256)
        return HP_ERR_ARG;
    if (!num_q_heads || num_q_heads % d->num_heads)
        return HP_ERR_ARG;
    // grid limits: grid x = units + num_seqs, grid y = head groups; Hq * D
    // indexes one sequence's output in 32 bits
    if (d->page_size > 65536 || d->num_seqs >= (1ull << 31) ||
        (uint64_t)num_q_heads * D >= (1ull << 31))
        return HP_ERR_ARG;
    for (int stream = 0; stream < 2; ++stream) {  // the launch shape may follow the hint
        const hp::AttentionShape sh =
            hp::attention_shape(d->num_seqs, d->total_tokens, d->page_size, d->num_heads, D,
                                num_q_heads, stream != 0, q8);
        if (sh.cap_units + d->num_seqs >= (1ull << 31) || sh.head_groups > 65535 ||
            (num_q_heads / d->num_heads + 7) / 8 > 65535)
            return HP_ERR_ARG;
    }
    return HP_OK;
}

size_t hp_attention_workspace_bytes(const hp_desc *desc, uint32_t num_q_heads) {
    Geometry g;
    if (!desc || check_desc(desc, &g) != HP_OK ||
        check_attention(desc, num_q_heads, desc->dtype == HP_DTYPE_I8) != HP_OK)
        return 0;
    return hp::attention_workspace_bytes(desc->num_seqs, desc->total_tokens, desc->page_size,
                                         desc->num_heads, desc->head_dim, num_q_heads);
}

// hp_paged_attention and hp_paged_attention_q8 (q8: int8 pools, the K
// scales in desc->scales, the V scales in v_scales).
static hp_status paged_attention(const hp_desc *desc, const void *v_pool,
                                 const float *v_scales, const void *q, uint32_t num_q_heads,
                                 float scale, void *out, uint32_t out_dtype, void *workspace,
                                 size_t workspace_bytes, uint32_t flags, void *stream, bool q8) {
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    if (out_dtype != HP_DTYPE_F32)
        return HP_ERR_DTYPE;
    if ((st = check_attention(desc, num_q_heads, q8)) != HP_OK)
        return st;
    if (flags & ~(uint32_t)(HP_FLAG_CHECKED | HP_FLAG_STREAM | HP_FLAG_PLANNED))
        return HP_ERR_ARG;
    const uint64_t S = desc->num_seqs, D = desc->head_dim;
    if (S && (!v_pool || !q || !out))
        return HP_ERR_NULL;
    if (q8 && S && (!desc->scales || !v_scales))
        return HP_ERR_NULL;
    if (!aligned(v_pool, 64) || !aligned(q, 16) || !aligned(out, 16) || !aligned(v_scales, 64))
        return HP_ERR_ALIGN;
    const uint64_t need = hp::attention_workspace_bytes(S, desc->total_tokens, desc->page_size,
                                                        desc->num_heads, D, num_q_heads);
    if ((st = check_workspace(workspace, workspace_bytes, need)) != HP_OK)
        return st;
    if (!aligned(workspace, 256))
        return HP_ERR_ALIGN;
    const uint64_t q_bytes = S * num_q_heads * D * 2, out_bytes = S * num_q_heads * D * 4;
    const uint64_t scale_bytes = q8 ? desc->num_pages * desc->page_size * 4 : 0;
    const void *reads[5] = {desc->page_pool, v_pool, q, desc->scales, v_scales};
    const uint64_t read_bytes[5] = {g.pool_bytes, g.pool_bytes, q_bytes, scale_bytes,
                                    scale_bytes};
    for (int i = 0; i < 5; ++i)
        if (overlaps(out, out_bytes, reads[i], read_bytes[i]) ||
            overlaps(workspace, need, reads[i], read_bytes[i]))
            return HP_ERR_ARG;
    if (overlaps(out, out_bytes, workspace, need))
        return HP_ERR_ARG;
    if (flags & HP_FLAG_CHECKED) {
        hp_validate_result r;
        if ((st = run_validate(desc, nullptr, workspace, &r, (hipStream_t)stream)) != HP_OK)
            return st;
    }
    if (!S)
        return HP_OK;
    hp::AttentionJob j = {};
    j.idx64 = desc->index_type == HP_INDEX_U64;
    j.bf16 = desc->dtype == HP_DTYPE_BF16 || q8;
    j.q8 = q8;
    j.planned = flags & HP_FLAG_PLANNED;
    j.stream_loads = flags & HP_FLAG_STREAM;
    j.num_seqs = (uint32_t)S;
    j.page_size = desc->page_size;
    j.num_kv_heads = desc->num_heads;
    j.num_q_heads = num_q_heads;
    j.head_dim = desc->head_dim;
    j.total_tokens = desc->total_tokens;
    j.k_pool = desc->page_pool;
    j.v_pool = v_pool;
    j.q = q;
    j.block_table = desc->block_table;
    j.seq_ptr = desc->seq_ptr;
    j.seq_lens = desc->seq_lens;
    if (q8) {
        j.k_scales = desc->scales;
        j.v_scales = v_scales;
    }
    j.out = static_cast<float *>(out);
    j.scale = scale;
    j.workspace = workspace;
    const hipError_t e = hp::launch_attention(j, (hipStream_t)stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

hp_status hp_attention_plan(const hp_desc *desc, uint32_t num_q_heads, void *workspace,
                            size_t workspace_bytes, uint32_t flags, void *stream) {
    Geometry g;
    hp_status st = check_desc(desc, &g);
    if (st != HP_OK)
        return st;
    const bool q8 = desc->dtype == HP_DTYPE_I8;
    if ((st = check_attention(desc, num_q_heads, q8)) != HP_OK)
        return st;
    if (flags & ~(uint32_t)(HP_FLAG_CHECKED | HP_FLAG_STREAM))
        return HP_ERR_ARG;
    const uint64_t S = desc->num_seqs;
    const uint64_t need = hp::attention_workspace_bytes(S, desc->total_tokens, desc->page_size,
                                                        desc->num_heads, desc->head_dim,
                                                        num_q_heads);
    if ((st = check_workspace(workspace, workspace_bytes, need)) != HP_OK)
        return st;
    if (!aligned(workspace, 256))
        return HP_ERR_ALIGN;
    if (flags & HP_FLAG_CHECKED) {
        hp_validate_result r;
        if ((st = run_validate(desc, nullptr, workspace, &r, (hipStream_t)stream)) != HP_OK)
            return st;
    }
    if (!S)
        return HP_OK;
    hp::AttentionJob j = {};
    j.idx64 = desc->index_type == HP_INDEX_U64;
    j.bf16 = desc->dtype == HP_DTYPE_BF16 || q8;
    j.q8 = q8;
    j.stream_loads = flags & HP_FLAG_STREAM;
    j.num_seqs = (uint32_t)S;
    j.page_size = desc->page_size;
    j.num_kv_heads = desc->num_heads;
    j.num_q_heads = num_q_heads;
    j.head_dim = desc->head_dim;
    j.total_tokens = desc->total_tokens;
    j.block_table = desc->block_table;
    j.seq_ptr = desc->seq_ptr;
    j.seq_lens = desc->seq_lens;
    j.workspace = workspace;
    const hipError_t e = hp::launch_attention_plan(j, (hipStream_t)stream);
    return e == hipSuccess ? HP_OK : hip_failed(e);
}

hp_status hp_paged_attention(const hp_desc *desc, const void *v_pool, const void *q,
                             uint32_t num_q_heads, float scale, void *out, uint32_t out_dtype,
                             void *workspace, size_t workspace_bytes, uint32_t flags,
                             void *stream) {
    return paged_attention(desc, v_pool, nullptr, q, num_q_heads, scale, out, out_dtype,
                           workspace, workspace_bytes, flags, stream, false);
}

hp_status hp_paged_attention_q8(const hp_desc *desc, const void *v_pool, const float *v_scales,
                                const void *q, uint32_t num_q_heads, float scale, void *out,
                                uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream) {
    return paged_attention(desc, v_pool, v_scales, q, num_q_heads, scale, out, out_dtype,
                           workspace, workspace_bytes, flags, stream, true);
}

hp_status hp_copy_pages(const hp_desc *desc, const void *src_pages, const void *dst_pages,
                        uint64_t count, void *workspace, size_t workspace_bytes, uint32_t flags,
                        void *stream) {
    if (!desc)
        return HP_ERR_NULL;
    void *pool = desc->page_pool;
    float *scales = const_cast<float *>(desc->scales);  // written by this call
    return copy_pages_common(desc, 1, &pool, desc->scales ? &scales : nullptr, src_pages,
                             dst_pages, count, workspace, workspace_bytes, flags,
                             (hipStream_t)stream);
}

hp_status hp_copy_pages_batch(const hp_desc *desc, uint32_t num_pools, void *const *pools,
                              float *const *scales, const void *src_pages, const void *dst_pages,
                              uint64_t count, void *workspace, size_t workspace_bytes,
                              uint32_t flags, void *stream) {
    return copy_pages_common(desc, num_pools, pools, scales, src_pages, dst_pages, count,
                             workspace, workspace_bytes, flags, (hipStream_t)stream);
}

const char *hp_last_hip_error(void) { return hipGetErrorName(t_last_hip_error); }

const char *hp_status_str(int status) {
    switch (status) {
    case HP_OK: return "HP_OK";
    case HP_ERR_NULL: return "HP_ERR_NULL: a required pointer is NULL";
    case HP_ERR_ARG: return "HP_ERR_ARG: invalid size, field or flag";
    case HP_ERR_RANK: return "HP_ERR_RANK: block-paged requires rank 3";
    case HP_ERR_PAGED_AXIS: return "HP_ERR_PAGED_AXIS: paged_axis must be 0";
    case HP_ERR_INDEX_TYPE: return "HP_ERR_INDEX_TYPE: unknown or too narrow index type";
    case HP_ERR_DTYPE: return "HP_ERR_DTYPE: unsupported element type";
    case HP_ERR_ALIGN: return "HP_ERR_ALIGN: buffer misaligned";
    case HP_ERR_WORKSPACE: return "HP_ERR_WORKSPACE: workspace missing or too small";
    case HP_ERR_SHARDED: return "HP_ERR_SHARDED: block-paged tensors cannot be sharded";
    case HP_ERR_QUANT: return "HP_ERR_QUANT: quantization scheme not accepted on block-paged";
    case HP_ERR_SEQPTR_FIRST: return "HP_ERR_SEQPTR_FIRST: seq_ptr[0] != 0";
    case HP_ERR_SEQPTR_LAST: return "HP_ERR_SEQPTR_LAST: seq_ptr[num_seqs] != block_table length";
    case HP_ERR_SEQPTR_ORDER: return "HP_ERR_SEQPTR_ORDER: seq_ptr decreases";
    case HP_ERR_PAGE_RANGE: return "HP_ERR_PAGE_RANGE: page ID out of range";
    case HP_ERR_SEQ_LEN: return "HP_ERR_SEQ_LEN: token count exceeds the sequence's pages";
    case HP_ERR_TOTAL_TOKENS: return "HP_ERR_TOTAL_TOKENS: seq_lens do not sum to total_tokens";
    case HP_ERR_WRITE_ALIAS: return "HP_ERR_WRITE_ALIAS: a scatter would write a slot twice";
    case HP_ERR_HIP: return "HP_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown hp_status";
    }
}

} // extern "C"
