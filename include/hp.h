/*
 * hp.h -- block-paged KV layout on MI355X (gfx950): gather, scatter,
 * dequant-gather and storage-invariant validation through a block table.
 *
 * The layout is the one defined by "Block-Paged Layout -- Hurray Format
 * Specification" (cited below as [Hurray]): a shared page pool
 * [num_pages, page_size, num_heads, head_dim], a block table of physical page
 * IDs, and a CSR offset array seq_ptr delimiting each sequence's slice of the
 * block table. The logical tensor is the ragged [total_tokens, num_heads,
 * head_dim] tensor whose rows are the sequences' tokens, sequence after
 * sequence, each in token order ([Hurray] Logical Shape).
 *
 * Element lookup ([Hurray] Element Lookup), for token t of sequence s:
 *   phys_page = block_table[seq_ptr[s] + t / page_size]
 *   flat      = ((phys_page*page_size + t % page_size)*num_heads + h)*head_dim + d
 *
 * Conventions shared by every call:
 *   - Every buffer pointer is a DEVICE pointer unless stated otherwise, owned
 *     by the caller. The library allocates nothing, frees nothing, keeps no
 *     pointer after a call returns and holds no global mutable state; calls
 *     are thread-safe.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on
 *     it; buffers are read and written when the stream reaches that work.
 *   - Argument errors are detected on the host before anything is enqueued:
 *     on any non-HP_OK return nothing has been written.
 *   - gather / scatter / gather_dequant are permissive readers ([Hurray]
 *     Storage Invariants permits a permissive mode): they trust the data
 *     invariants unless HP_FLAG_CHECKED is given, in which case hp_validate
 *     runs first (synchronously) and its code is returned without writing;
 *     with HP_FLAG_GATED the device checks the verdict of an earlier
 *     hp_validate_async on the same workspace and writes nothing on a
 *     violation, with no host wait. Unchecked calls on a descriptor that
 *     violates (1)-(3) or the token-count bound have undefined results.
 *   - An empty batch (num_seqs = 0, seq_ptr = [0], block_table may be NULL;
 *     [Hurray] Buffer Table note) is valid; calls on it enqueue nothing.
 */
#ifndef HP_H
#define HP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. No call throws; every call returns one of these. */
typedef enum hp_status {
    HP_OK = 0,
    HP_ERR_NULL = 1,          /* a required pointer is NULL */
    HP_ERR_ARG = 2,           /* zero page_size/num_heads/head_dim, size overflow,
                                 byte_offset != 0, reserved field != 0, bad flag */
    HP_ERR_RANK = 3,          /* rank != 3 ([Hurray] Description) */
    HP_ERR_PAGED_AXIS = 4,    /* paged_axis != 0 ([Hurray] Logical Shape, invariant 6) */
    HP_ERR_INDEX_TYPE = 5,    /* unknown index type, or uint32 too narrow
                                 ([Hurray] Additional Descriptor Fields note) */
    HP_ERR_DTYPE = 6,         /* unknown or unsupported element type */
    HP_ERR_ALIGN = 7,         /* descriptor buffer not 64-byte aligned ([Hurray]
                                 Alignment) or other buffer not element aligned */
    HP_ERR_WORKSPACE = 8,     /* workspace NULL or smaller than hp_workspace_bytes */
    HP_ERR_SHARDED = 9,       /* a shard descriptor is attached ([Hurray] Sharding) */
    HP_ERR_QUANT = 10,        /* quantization scheme a block-paged reader must reject
                                 ([Hurray] Per-scheme composition) */
    HP_ERR_SEQPTR_FIRST = 16, /* seq_ptr[0] != 0                     (invariant 1) */
    HP_ERR_SEQPTR_LAST = 17,  /* seq_ptr[num_seqs] != num_block_entries (invariant 1) */
    HP_ERR_SEQPTR_ORDER = 18, /* seq_ptr[s] > seq_ptr[s+1]           (invariant 2) */
    HP_ERR_PAGE_RANGE = 19,   /* block_table[k] >= num_pages         (invariant 3) */
    HP_ERR_SEQ_LEN = 20,      /* seq_start[s] + seq_lens[s] > slice pages * page_size
                                 ([Hurray] Partial trailing page: reads and writes
                                 are bounded by the slice and the token count) */
    HP_ERR_TOTAL_TOKENS = 21, /* sum of seq_lens != total_tokens ([Hurray] Logical Shape) */
    HP_ERR_WRITE_ALIAS = 22,  /* a scatter would write one slot more than once
                                 ([Hurray] Prefix Sharing; HP_FLAG_DISJOINT) */
    HP_ERR_HIP = 32           /* a HIP runtime call or kernel launch failed */
} hp_status;

/* block_table_index_type ([Hurray] Additional Descriptor Fields, Example):
 * element type of block_table, seq_ptr, seq_lens and seq_start. */
enum { HP_INDEX_U32 = 0x00, HP_INDEX_U64 = 0x01 };

/* Element types of page_pool / the logical tensor. Gather and scatter are bit
 * copies, so only the width matters to them. */
enum {
    HP_DTYPE_I8 = 1, HP_DTYPE_U8 = 2, HP_DTYPE_F16 = 3, HP_DTYPE_BF16 = 4,
    HP_DTYPE_F32 = 5, HP_DTYPE_F64 = 6
};

/* Flags. */
enum {
    HP_FLAG_CHECKED = 1u << 0,   /* validate first; on a violation write nothing */
    HP_FLAG_ZERO_TAIL = 1u << 1, /* scatter: zero the slots of each sequence's last
                                    written page past its last new token ([Hurray]
                                    Partial trailing page: a writer should zero them) */
    HP_FLAG_STREAM = 1u << 2,    /* gather: performance hint that no pool page is read
                                    twice by this call (the slices do not alias, [Hurray]
                                    Prefix Sharing); the pool is then read with
                                    non-temporal loads. Results are identical with or
                                    without it; with aliased pages it is only slower. */
    HP_FLAG_GATED = 1u << 3,     /* gather, scatter, dequant-gather and their batched and
                                    quantized forms: the verdict that hp_validate_async
                                    left in the head of `workspace` decides, on the
                                    device, whether the call writes anything (see
                                    hp_validate_async). Not combined with
                                    HP_FLAG_CHECKED. */
    HP_FLAG_DISJOINT = 1u << 4,  /* scatter, quantize-on-scatter and the batched
                                    scatter, with HP_FLAG_CHECKED only: after the
                                    descriptor passes validation, also check that no
                                    slot is written twice (hp_validate_writes); on a
                                    clash return HP_ERR_WRITE_ALIAS and write nothing.
                                    The workspace must hold
                                    hp_disjoint_workspace_bytes(desc). */
    HP_FLAG_PLANNED = 1u << 5    /* attention: the workspace already holds the plan
                                    hp_attention_plan wrote for this descriptor
                                    (table, counts, total_tokens unchanged since),
                                    num_q_heads and HP_FLAG_STREAM setting, so the
                                    call runs no planning kernel (one plan serves the
                                    calls of every layer of one batch); results are
                                    undefined if the plan is stale. */
};

/* A block-paged descriptor for one {kv_role, layer_index} pair ([Hurray]
 * Description, Buffer Table, Additional Descriptor Fields, Example).
 * Host memory; read during the call only. */
typedef struct hp_desc {
    uint32_t rank;              /* must be 3 */
    uint32_t paged_axis;        /* must be 0 */
    uint32_t index_type;        /* HP_INDEX_U32 or HP_INDEX_U64 */
    uint32_t dtype;             /* HP_DTYPE_* of page_pool elements */
    uint32_t page_size;         /* P > 0 (tokens per page) */
    uint32_t num_heads;         /* H > 0 */
    uint32_t head_dim;          /* D > 0 */
    uint32_t has_shard;         /* must be 0: block-paged may not be sharded */
    uint32_t kv_role;           /* informational (0 key, 1 value); not read */
    uint32_t layer_index;       /* informational; not read */
    uint64_t byte_offset;       /* must be 0 ([Hurray] byte_offset) */
    uint64_t num_pages;         /* N: pages in page_pool */
    uint64_t num_seqs;          /* S */
    uint64_t num_block_entries; /* K: entries in block_table (total_logical_pages) */
    uint64_t total_tokens;      /* T: rows of the logical tensor = sum of seq_lens */
    void *page_pool;            /* buffer 0: N*P*H*D elements, 64-byte aligned;
                                   written only by hp_scatter */
    const void *block_table;    /* buffer 1: K page IDs (index_type), 64-byte
                                   aligned; may be NULL when K == 0 */
    const void *seq_ptr;        /* buffer 2: S+1 offsets (index_type), 64-byte aligned */
    const void *seq_lens;       /* S token counts (index_type); NULL allowed if S == 0 */
    const float *scales;        /* buffer 3 (quantized pools only): N*P fp32, one per
                                   page slot ([Hurray] Per-page-slot parameters),
                                   64-byte aligned; NULL otherwise */
} hp_desc;

/* Result of hp_validate, written to HOST memory. */
typedef struct hp_validate_result {
    int32_t code;      /* HP_OK or the first failing HP_ERR_* */
    uint32_t reserved;
    uint64_t index;    /* smallest failing s or k for that check; num_seqs for
                          HP_ERR_SEQPTR_LAST; 0 otherwise */
} hp_validate_result;

/* Bytes of device workspace (any alignment >= 256 is fine) that any call on
 * `desc` needs; 0 if none. Returns 0 for an invalid descriptor too (the call
 * itself reports the error). */
size_t hp_workspace_bytes(const hp_desc *desc);

/* Storage-invariant validator ([Hurray] Storage Invariants: a reader should
 * validate (1)-(3) and (6) and must reject violations).
 * Host-side: rank, paged_axis, shard, sizes. Device-side, one parallel pass:
 * (1) seq_ptr[0] = 0 and seq_ptr[S] = K; (2) seq_ptr non-decreasing;
 * (3) block_table[k] < N; then the token-count bound
 *     seq_start[s] + seq_lens[s] <= (seq_ptr[s+1] - seq_ptr[s]) * P
 * (seq_start NULL means all starts are 0; pass the scatter's seq_start to
 * check a scatter's windows); then sum(seq_lens) = T.
 * The first failing check in that order is reported, with its smallest
 * failing index, so the result is deterministic. Aliased page IDs are
 * allowed ([Hurray] Prefix Sharing) and not checked.
 * Synchronous: enqueues on `stream`, brings 16 bytes back into *result and
 * waits for the stream. `result` is a host pointer and may be NULL. In pinned
 * host memory (hipHostMalloc) a descriptor of at most 65,536 items (table
 * entries or sequences) is checked by one workgroup that writes the result
 * there itself, with no copy; otherwise the words are copied from the
 * workspace. Returns result->code. */
hp_status hp_validate(const hp_desc *desc, const void *seq_start, void *workspace,
                      size_t workspace_bytes, hp_validate_result *result,
                      void *stream);

/* Enqueue-only validation ([Hurray] Storage Invariants: a reader validates
 * (1)-(3) and (6) and rejects a descriptor that violates them). The checks,
 * their order and the first-failure rule are those of hp_validate, and the
 * host checks happen the same way (rank, paged_axis, shard, sizes, with the
 * same error codes), but nothing waits: the device leaves its verdict, two
 * 64-bit words (the smallest failing (check, index) key, all ones when no
 * check failed, and the sum of seq_lens), in bytes [0, 16) of `workspace`
 * when `stream` reaches the work.
 *
 * A later move on the same workspace with HP_FLAG_GATED, ordered after this
 * call (same stream, or an event), reads the words on the device and writes
 * nothing at all (no output row, pool slot, scale or zero point) unless no
 * check failed and the sum equals that move's total_tokens. So "a rejected
 * descriptor is never moved" holds with no host round trip between batches.
 * The host learns the verdict only if it asks: copy the 16 bytes back and
 * pass them to hp_validate_verdict.
 *
 * workspace  DEVICE, 8-byte aligned, at least 256 bytes (hp_workspace_bytes
 *            of the moves covers it); the words stay there until the next
 *            validation on that workspace. Moves read the head only when
 *            gated. A gated move with no validation before it on its
 *            workspace reads whatever the head holds.
 * seq_start  as in hp_validate (NULL: all starts 0; pass a scatter's starts
 *            to check its windows).
 * Returns HP_OK once enqueued, a host-side argument error, or HP_ERR_HIP. */
hp_status hp_validate_async(const hp_desc *desc, const void *seq_start, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Bytes of device workspace that hp_validate_writes, and a scatter with
 * HP_FLAG_DISJOINT, need on `desc`: 512 plus two bitmaps of num_pages *
 * page_size bits, and at least hp_workspace_bytes(desc). 0 for an invalid
 * descriptor. */
size_t hp_disjoint_workspace_bytes(const hp_desc *desc);

/* Write-disjointness of a scatter ([Hurray] Prefix Sharing: slices may name
 * the same page, so two written rows, or a row and a zeroed tail slot of
 * [Hurray] Partial trailing page, can land in one slot, and a scatter is
 * defined only when they do not). First the checks of hp_validate, with
 * seq_start; if they pass, the slots the scatter would write (token
 * seq_start[s] + i of sequence s for i < seq_lens[s] and, with
 * HP_FLAG_ZERO_TAIL in `flags`, the slots of the last token's page after it)
 * are marked in a bitmap over the pool's slots. HP_ERR_WRITE_ALIAS is
 * reported with index = the smallest sequence one of whose written slots is
 * written more than once (by any sequence, itself included); HP_OK when every
 * written slot is written once. Deterministic.
 * Synchronous, like hp_validate: enqueues on `stream`, waits, writes *result
 * (HOST, may be NULL) and returns result->code. workspace: DEVICE, 8-byte
 * aligned, at least hp_disjoint_workspace_bytes(desc). flags: 0 or
 * HP_FLAG_ZERO_TAIL. */
hp_status hp_validate_writes(const hp_desc *desc, const void *seq_start, uint32_t flags,
                             void *workspace, size_t workspace_bytes,
                             hp_validate_result *result, void *stream);

/* Decodes the 16 verdict bytes of hp_validate_async (`words`, HOST memory,
 * e.g. copied back from the workspace head) into *result, exactly as
 * hp_validate reports it, for the descriptor's total_tokens. Returns
 * result->code; HP_ERR_NULL if a pointer is NULL. Host only. */
hp_status hp_validate_verdict(const hp_desc *desc, const void *words,
                              hp_validate_result *result);

/* Gather ([Hurray] Element Lookup, Logical Shape): writes the logical tensor
 *   out[(sum_{s'<s} seq_lens[s']) + t][h][d] = page_pool[flat(s, t, h, d)]
 * for every s < S, t < seq_lens[s], as a bit copy. `out` is a device buffer
 * of T*H*D elements of desc->dtype, element aligned, not overlapping
 * page_pool. No slot at or past a sequence's token count is read ([Hurray]
 * Partial trailing page). Slices may alias pages. Asynchronous.
 * Flags: HP_FLAG_CHECKED or HP_FLAG_GATED, HP_FLAG_STREAM. */
hp_status hp_gather(const hp_desc *desc, void *out, void *workspace,
                    size_t workspace_bytes, uint32_t flags, void *stream);

/* Gather for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * same move, flags and results as hp_gather, with no workspace argument: the
 * workspace is a library-owned device array of about 3 MiB (each GPU the
 * library runs on holds its own copy until the process ends). It holds the
 * validator's words (HP_FLAG_CHECKED) and the plan arrays of calls over many
 * sequences, at most 262,144 sequences (more: HP_ERR_WORKSPACE, nothing
 * enqueued). The call allocates and frees nothing.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (everything a call reads there it first writes): calls
 * that overlap on one GPU (concurrent streams, or host threads on one
 * device) race and must not be made. `stream` must belong to the current
 * device. Flags: HP_FLAG_CHECKED (synchronous, as in hp_gather),
 * HP_FLAG_STREAM; HP_FLAG_GATED is rejected (HP_ERR_ARG), as is everything
 * hp_gather rejects. */
hp_status hp_gather_static(const hp_desc *desc, void *out, uint32_t flags, void *stream);

/* Scatter: the inverse move. `src` holds T = sum(seq_lens) new rows
 * [T, H, D] of desc->dtype in logical order; the i-th new row of sequence s
 * is token seq_start[s] + i of that sequence and is written to
 *   page_pool[flat(s, seq_start[s] + i, h, d)]
 * (seq_start: S device entries of index_type, or NULL for all zeros).
 * With HP_FLAG_ZERO_TAIL and seq_lens[s] > 0, the slots of the page holding
 * the last new token that come after it are set to zero bytes ([Hurray]
 * Partial trailing page). Destinations of different rows must be distinct
 * slots (aliased pages must be copied before they are written); otherwise
 * the result is undefined (HP_FLAG_DISJOINT checks it). Asynchronous.
 * Flags: HP_FLAG_CHECKED (validates with seq_start; with HP_FLAG_DISJOINT
 * also the distinct destinations) or HP_FLAG_GATED, HP_FLAG_ZERO_TAIL. */
hp_status hp_scatter(const hp_desc *desc, const void *src, const void *seq_start,
                     void *workspace, size_t workspace_bytes, uint32_t flags,
                     void *stream);

/* Dequant-gather ([Hurray] Element Lookup, Per-page-slot parameters): for an
 * int8 pool (desc->dtype = HP_DTYPE_I8) with per-slot scales (desc->scales),
 *   out[row][h][d] = bf16_rne( fp32(q) * scales[phys_page*P + t % P] )
 * one IEEE binary32 multiply, then round to nearest even into bfloat16; rows
 * as in hp_gather. out_dtype must be HP_DTYPE_BF16; `out` holds T*H*D bf16
 * values, 2-byte aligned. Asynchronous. Flags: HP_FLAG_CHECKED or HP_FLAG_GATED. */
hp_status hp_gather_dequant(const hp_desc *desc, void *out, uint32_t out_dtype,
                            void *workspace, size_t workspace_bytes, uint32_t flags,
                            void *stream);

/* ---- Quantize-on-scatter ----------------------------------------------------
 *
 * [Hurray] Per-page-slot parameters: a quantized page carries one scale (and,
 * for an asymmetric scheme, one zero point) per physical slot. This is the
 * scatter of hp_scatter for a quantized pool: each new token's row of
 * num_heads * head_dim values is quantized on its own and its codes, scale
 * and zero point are written to its slot. The formulas belong to a scheme
 * document that is not given; the reading used (each step one IEEE binary32
 * operation, round to nearest even):
 *   int8 pool (symmetric, zero_points NULL):
 *     scale = max|x| / 127, q = clamp(rint(x / scale), -127, 127)
 *   uint8 pool (asymmetric, zero_points required):
 *     lo = min(0, min x), hi = max(0, max x), scale = (hi - lo) / 255,
 *     z = clamp(rint(-lo / scale), 0, 255), q = clamp(rint(x / scale) + z, 0, 255)
 * and a zero scale gives zero codes and zero point. Rows holding NaN or an
 * infinity get unspecified codes. hp_gather_dequant_q with the
 * per-block-affine scheme (or hp_gather_dequant for int8) reads them back.
 *
 * desc        the quantized pool (dtype HP_DTYPE_I8 or HP_DTYPE_U8); desc->scales
 *             (fp32, num_pages * page_size) is WRITTEN at every written slot.
 * src         DEVICE [total_tokens, num_heads, head_dim] of src_dtype
 *             (HP_DTYPE_F16, HP_DTYPE_BF16 or HP_DTYPE_F32), element aligned.
 * zero_points DEVICE uint8 [num_pages * page_size], 64-byte aligned (uint8 pools).
 * seq_start, workspace, flags (HP_FLAG_CHECKED, with HP_FLAG_DISJOINT, or
 * HP_FLAG_GATED; HP_FLAG_ZERO_TAIL: tail slots get zero codes, scale 0 and zero
 * point 0) and errors as hp_scatter. */
hp_status hp_scatter_quant(const hp_desc *desc, const void *src, uint32_t src_dtype,
                           void *zero_points, const void *seq_start, void *workspace,
                           size_t workspace_bytes, uint32_t flags, void *stream);

/* ---- Dequant-gather under any quantization scheme -------------------------
 *
 * [Hurray] Quantization Compatibility, Per-scheme composition. Schemes, by the
 * spec's scheme tags, and where the parameter of element (t, h, d) of
 * sequence s lives:
 *   HP_QUANT_PER_TENSOR (0x01)        scales[0]
 *   HP_QUANT_PER_CHANNEL (0x02)       axis 1: scales[h] (num_heads entries);
 *                                     axis 2: scales[d] (head_dim entries);
 *                                     axis 0 (the paged axis) is rejected
 *   HP_QUANT_PER_BLOCK_AFFINE (0x03)  axis 0 and block_size == page_size only:
 *                                     scales[phys_page*page_size + t % page_size]
 * and likewise zero_points (NULL: symmetric). The pool is int8 (HP_DTYPE_I8)
 * or uint8 (HP_DTYPE_U8); zero points have the pool's element type. Each
 * output element is
 *   bf16_rne( fp32(q - zp) * scale )
 * with q - zp exact in integers and one IEEE binary32 multiply (the formulas
 * of the scheme document the spec defers to are not given; this affine form
 * with the symmetric case zp = 0 is the reading used). A rejected scheme
 * returns HP_ERR_QUANT. desc->scales is not used. scales and zero_points are
 * DEVICE buffers, 64-byte aligned. Other arguments as hp_gather_dequant. */
enum { HP_QUANT_PER_TENSOR = 0x01, HP_QUANT_PER_CHANNEL = 0x02, HP_QUANT_PER_BLOCK_AFFINE = 0x03 };

typedef struct hp_quant {
    uint32_t scheme;          /* HP_QUANT_* */
    uint32_t axis;            /* 1 or 2 for per-channel; 0 for per-block-affine */
    uint64_t block_size;      /* per-block-affine: must equal page_size */
    const float *scales;      /* device; count as listed above */
    const void *zero_points;  /* device, or NULL for a symmetric scheme */
} hp_quant;

hp_status hp_gather_dequant_q(const hp_desc *desc, const hp_quant *quant, void *out,
                              uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                              uint32_t flags, void *stream);

/* ---- Batched moves over pools that share one block table ------------------
 *
 * [Hurray] Description: a whole KV cache ([layers, 2, ...]) travels as a
 * stream of descriptors, one per {kv_role, layer_index}; in a paged cache all
 * of them use the same block table, seq_ptr and token counts and differ only
 * in their page pool (and scales). A batched call moves `count` such pools in
 * one pass over the table: member i uses pools[i] (and scales[i]) with the
 * geometry and index buffers of `desc`, whose own page_pool and scales fields
 * are ignored. The result for member i is exactly that of the single call on
 * the descriptor with page_pool = pools[i] (scales = scales[i]).
 *
 * pools, outs, srcs and scales are HOST arrays of `count` DEVICE pointers.
 * Every pool is 64-byte aligned; outputs are element aligned (bf16 for
 * dequant). No output overlaps any pool, scale buffer or another output; for
 * scatter the pools do not overlap each other. count == 0 enqueues nothing.
 * Flags, workspace and errors are those of the single calls. */
hp_status hp_gather_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                          void *const *outs, void *workspace, size_t workspace_bytes,
                          uint32_t flags, void *stream);

hp_status hp_scatter_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                           const void *const *srcs, const void *seq_start, void *workspace,
                           size_t workspace_bytes, uint32_t flags, void *stream);

hp_status hp_gather_dequant_batch(const hp_desc *desc, uint32_t count, void *const *pools,
                                  const float *const *scales, void *const *outs,
                                  uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                                  uint32_t flags, void *stream);

/* ---- Copy-on-write page copy -----------------------------------------------
 *
 * [Day51] "Copy-on-write for beam search and prefix sharing": pages shared by
 * several sequences ([Hurray] Prefix Sharing) are copied before one of them
 * writes into it; [Hurray] Per-page-slot parameters: a page carries its own
 * slot scales. For i < count, page dst_pages[i] of the pool becomes a copy of
 * page src_pages[i] (all page_size * num_heads * head_dim elements), and, when
 * the pool has scales, scales[dst*P .. dst*P+P) become those of src.
 *
 * src_pages / dst_pages: `count` DEVICE page IDs of desc->index_type. The
 * destinations must be distinct and must not be sources of the same call
 * (otherwise the result depends on scheduling). Only the pool (and its
 * scales) is read and written; block_table / seq_ptr / seq_lens are not used.
 * Asynchronous. Flags: HP_FLAG_CHECKED checks that every page ID is below
 * num_pages (HP_ERR_PAGE_RANGE otherwise; workspace >= 256 bytes needed). */
hp_status hp_copy_pages(const hp_desc *desc, const void *src_pages, const void *dst_pages,
                        uint64_t count, void *workspace, size_t workspace_bytes, uint32_t flags,
                        void *stream);

/* The same copies in `num_pools` pools at once (every layer and role of a KV
 * cache names a page by the same ID): pools and scales are HOST arrays of
 * `num_pools` DEVICE pointers (scales may be NULL, or hold NULLs); the pools
 * must not overlap. desc's own page_pool and scales are ignored. */
hp_status hp_copy_pages_batch(const hp_desc *desc, uint32_t num_pools, void *const *pools,
                              float *const *scales, const void *src_pages, const void *dst_pages,
                              uint64_t count, void *workspace, size_t workspace_bytes,
                              uint32_t flags, void *stream);

/* ---- Decode attention through the block table ------------------------------
 *
 * [Day51] "How the attention kernel uses the block table": attention reads a
 * sequence's keys and values block by block through its table; [Rust20]
 * "Keep token order across cache pages": paging changes where rows are
 * stored, not the dot products or the weighted sums. For sequence s and query
 * head hq, with G = num_q_heads / num_heads query heads per kv head and kv
 * head h = hq / G,
 *   x_t = scale * sum_d q[s][hq][d] * K[t][h][d]
 *   out[s][hq][d] = sum_t exp(x_t) * V[t][h][d] / sum_t exp(x_t)
 * over the L_s = seq_lens[s] cached tokens t, whose K and V rows sit at
 * [Hurray] Element Lookup's position in the two pools. A sequence with no
 * tokens gives zeros.
 *
 * desc      the K cache: its page_pool is the K pool; num_heads is the number
 *           of kv heads; dtype HP_DTYPE_F16 or HP_DTYPE_BF16; head_dim one of
 *           8, 16, 32, 64, 128, 256; page_size at most 65,536; total_tokens
 *           must be the sum of the counts (it sizes the grid and workspace).
 * v_pool    DEVICE, the V pool: same geometry, dtype and block table as K
 *           ([Hurray] Description: one descriptor per kv_role), 64-byte aligned.
 * q         DEVICE [num_seqs, num_q_heads, head_dim] of the pool's dtype,
 *           16-byte aligned.
 * num_q_heads  a multiple G of num_heads (any G >= 1).
 * scale     the softmax scale (1/sqrt(head_dim) in the usual form).
 * out       DEVICE [num_seqs, num_q_heads, head_dim] fp32 (out_dtype
 *           HP_DTYPE_F32), 16-byte aligned.
 * workspace DEVICE, 256-byte aligned, at least
 *           hp_attention_workspace_bytes(desc, num_q_heads) bytes (per-unit
 *           partial results); it may not overlap any other buffer.
 * Arithmetic is fp32 with an online softmax in base 2; the result differs
 * from the exact one by rounding only. Flags: HP_FLAG_CHECKED (validate
 * first), HP_FLAG_STREAM (no page is read twice in this call: non-temporal
 * loads), HP_FLAG_PLANNED (reuse the plan of hp_attention_plan). Asynchronous
 * on `stream`. */
hp_status hp_paged_attention(const hp_desc *desc, const void *v_pool, const void *q,
                             uint32_t num_q_heads, float scale, void *out, uint32_t out_dtype,
                             void *workspace, size_t workspace_bytes, uint32_t flags,
                             void *stream);

/* Decode attention over int8 K and V pools with one fp32 scale per slot.
 *
 * [Hurray] Per-page-slot parameters: the scale of a slot sits at
 * scales[phys_page * page_size + t % page_size] and applies to every element
 * of that slot's row, whose value is code * scale. This call computes
 * hp_paged_attention's result over those values, with K[t] = cK_t * sK_t and
 * V[t] = cV_t * sV_t:
 *   x_t = (scale * sK_t) * sum_d q[s][hq][d] * cK_t[h][d]
 *   out[s][hq][d] = sum_t (e^{x_t} sV_t) cV_t[h][d] / sum_t e^{x_t}
 * in fp32 (the codes are exact in bf16, the queries bf16), so the result
 * differs from the exact one by fp32 rounding only. With power-of-two scales
 * it equals hp_paged_attention over bf16 pools holding code * scale bit for
 * bit (hp_gather_dequant writes such pools).
 *
 * desc      the K cache: dtype HP_DTYPE_I8, its page_pool the int8 K pool and
 *           its scales the K scales (num_pages * page_size fp32, 64-byte
 *           aligned); other requirements as hp_paged_attention.
 * v_pool    DEVICE, the int8 V pool: same geometry and block table as K,
 *           64-byte aligned.
 * v_scales  DEVICE, num_pages * page_size fp32 scales of the V pool, 64-byte
 *           aligned.
 * q         DEVICE [num_seqs, num_q_heads, head_dim] bf16, 16-byte aligned.
 * The other arguments, the workspace (hp_attention_workspace_bytes with
 * this descriptor), the flags and the errors are those of
 * hp_paged_attention; NULL scales with a non-empty batch give HP_ERR_NULL,
 * and neither out nor the workspace may overlap a scale buffer. */
hp_status hp_paged_attention_q8(const hp_desc *desc, const void *v_pool, const float *v_scales,
                                const void *q, uint32_t num_q_heads, float scale, void *out,
                                uint32_t out_dtype, void *workspace, size_t workspace_bytes,
                                uint32_t flags, void *stream);

/* The planning kernels of hp_paged_attention / hp_paged_attention_q8 alone,
 * into the workspace: for a batch whose sequences share leading pages
 * ([Hurray] Prefix Sharing) the comparison of neighbouring slices and the
 * shared-prefix plan, and above 4,096 sequences the unit plan; for other
 * shapes nothing. The plan depends only on the table, the counts, the launch
 * shape (num_q_heads, head_dim, the pool's element type and HP_FLAG_STREAM),
 * not on the pools or queries, so the attention calls of every layer of one
 * batch can pass HP_FLAG_PLANNED and reuse it.
 * desc         as for the attention call (its dtype picks the int8 shape).
 * workspace    DEVICE, 256-byte aligned, hp_attention_workspace_bytes bytes;
 *              the later calls must pass the same workspace.
 * flags        HP_FLAG_STREAM as the later calls will pass it; HP_FLAG_CHECKED
 *              validates the descriptor first (synchronously).
 * Asynchronous on `stream`. */
hp_status hp_attention_plan(const hp_desc *desc, uint32_t num_q_heads, void *workspace,
                            size_t workspace_bytes, uint32_t flags, void *stream);

/* Workspace bytes hp_paged_attention (f16 or bf16 pools) or
 * hp_paged_attention_q8 (int8 pools) needs for this descriptor (its
 * num_seqs, total_tokens and geometry); 0 for an invalid descriptor or an
 * unsupported shape. */
size_t hp_attention_workspace_bytes(const hp_desc *desc, uint32_t num_q_heads);

/* Static, human-readable name of a status code. */
const char *hp_status_str(int status);

/* Name of the HIP error (e.g. "hipErrorInvalidValue") behind the calling
 * thread's most recent HP_ERR_HIP, or "hipSuccess" if it has had none. The
 * value is kept per thread. Static string; never NULL. */
const char *hp_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HP_H */
