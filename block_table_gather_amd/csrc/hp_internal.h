// hp_internal.h -- what the C-ABI layer (hp_api.cpp) hands to the kernel
// launchers (hp_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hp {

// Tuning constants; each can be overridden at build time (-DHP_...). Unit
// bytes are the target size of one work unit on its larger side; measured on
// MI355X (8 KB gather spans stream best, 5 % ahead of 16 KB on the decode
// batch; dequant and small scatters prefer 32 KB).
#ifndef HP_THREADS
#define HP_THREADS 256
#endif
#ifndef HP_GATHER_UNIT_BYTES
#define HP_GATHER_UNIT_BYTES 8192
#endif
// Every gather workgroup reads each sequence's count and seq_ptr (8 or 16
// bytes) in its fused scan, so a gather unit is at least this many bytes per
// sequence: the table reads stay near 1/16 of what a unit moves, or below
// (256 sequences: 16 KB units, 17 % faster than 8 KB on the prefix batch).
#ifndef HP_GATHER_UNIT_BYTES_PER_SEQ
#define HP_GATHER_UNIT_BYTES_PER_SEQ 64
#endif
#ifndef HP_SCATTER_UNIT_BYTES
#define HP_SCATTER_UNIT_BYTES 32768
#endif
#ifndef HP_DEQUANT_UNIT_BYTES
#define HP_DEQUANT_UNIT_BYTES 32768
#endif
#ifndef HP_GATHER_UNITS_PER_GROUP
#define HP_GATHER_UNITS_PER_GROUP 1
#endif
#ifndef HP_SCATTER_UNITS_PER_GROUP
#define HP_SCATTER_UNITS_PER_GROUP 2
#endif
// A scatter that moves at least this many bytes cannot stay resident in the
// 256 MB Infinity Cache (MALL): it streams its source with non-temporal loads
// in small units; smaller scatters (appends) read through the cache in larger
// units, which measured faster when their source is cache-resident.
#ifndef HP_SCATTER_STREAM_BYTES
#define HP_SCATTER_STREAM_BYTES (256ull << 20)
#endif
#ifndef HP_SCATTER_STREAM_UNIT_BYTES
#define HP_SCATTER_STREAM_UNIT_BYTES 8192
#endif
// Quantize-on-scatter: rows (slots of one page) per work unit; the
// workgroup's waves take them in turn. Four (one row per wave) measured 5 %
// ahead of 8 and 7 % ahead of 16 on the decode batch.
#ifndef HP_QUANT_UNIT_ROWS
#define HP_QUANT_UNIT_ROWS 4
#endif
#ifndef HP_QUANT_UNITS_PER_GROUP
#define HP_QUANT_UNITS_PER_GROUP 1
#endif
#ifndef HP_DEQUANT_UNITS_PER_GROUP
#define HP_DEQUANT_UNITS_PER_GROUP 1
#endif
// Sequences whose per-sequence offsets fit in LDS: up to this many, every
// workgroup rebuilds the offsets itself (one fused launch); beyond it a plan
// pass writes them to the workspace first.
#ifndef HP_FUSED_MAX_SEQS
#define HP_FUSED_MAX_SEQS 4096
#endif
constexpr uint64_t kFusedMaxSeqs = HP_FUSED_MAX_SEQS;
// From this many sequences on, the moves in HP_PLAN_OPS (a bit per Op) take
// the plan pass when the caller's workspace holds its arrays, even where the
// fused scan would fit: each workgroup of the fused path reads and scans every
// sequence's count (16 KB of metadata per 16 KB unit on the quantized batch's
// 1,024 sequences); the plan pass writes the offsets once and each workgroup
// binary-searches them. Measured on MI355X with cold caches: quantized-batch
// gather 601 -> 553 us; the prefix batch (256 sequences) 152 -> 194 us the
// other way, and the dequant 934 -> 955 us, so only the gather takes it.
#ifndef HP_PLAN_MIN_SEQS
#define HP_PLAN_MIN_SEQS 512
#endif
#ifndef HP_PLAN_OPS
#define HP_PLAN_OPS 1
#endif
constexpr uint64_t kPlanMinSeqs = HP_PLAN_MIN_SEQS;
constexpr uint32_t kThreads = HP_THREADS;     // threads per copy workgroup
constexpr uint32_t kPlanChunk = 2048;         // sequences per plan workgroup
constexpr uint32_t kMaxUnitsPerGroup = 16;
// Sequences a one-wave quantize-on-scatter workgroup scans from registers
// (64 lanes x 4): more would make every one-slot workgroup read the counts
// twice.
constexpr uint32_t kQuantWaveMaxSeqs = 256;
// Pools moved by one launch of a batched call (one grid row each); the
// pointers travel in the kernel arguments. Larger batches take more launches.
constexpr uint32_t kMaxBatch = 32;

enum class Op : int { Gather = 0, Scatter = 1, Dequant = 2, ScatterQuant = 3 };
// Moves that write the pool (and so take seq_start and tail zeroing).
constexpr bool writes_pool(Op op) { return op == Op::Scatter || op == Op::ScatterQuant; }

// Everything a copy launch needs; filled and checked on the host.
struct CopyJob {
    Op op;
    bool idx64;             // index type is uint64
    bool zero_tail;         // scatter only
    uint32_t elem_bytes;    // pool element width
    uint32_t page_size;     // P
    uint32_t rows_per_unit; // divides P
    uint32_t units_per_group;
    bool load_nt;           // stream the source with non-temporal loads
    uint64_t num_seqs;      // S
    uint64_t total_tokens;  // T
    uint64_t row_bytes;     // H*D*elem_bytes (pool side)
    uint64_t out_row_bytes; // logical-tensor side (dequant: H*D*2)
    uint64_t unit_bound;    // host upper bound on the number of work units
    const void *block_table;
    const void *seq_ptr;
    const void *seq_lens;
    const void *seq_start;  // scatter, may be null
    uint32_t count;         // pools moved (each with its own rows and scales)
    void *const *pools;     // [count] pools: gather/dequant read them, scatter writes
    void *const *rows;      // [count] logical tensors: gather/dequant write, scatter reads
    const float *const *scales;  // [count] per-slot scales (dequant), else null
    void *workspace;        // plan arrays (plan path)
    bool plan;              // take the plan path (always when num_seqs > kFusedMaxSeqs)
    uint32_t vec_bytes;     // widest vector width every span allows
    // Dequant under a general scheme (single pool): 0 = per-slot scales from
    // `scales` (the fast path when there is no zero point and q is signed),
    // 1 = per-tensor, 2 = per-head, 3 = per-head_dim parameters.
    bool quant_ext;
    uint32_t quant_mode;
    bool quant_unsigned;    // uint8 pool (else int8)
    const float *quant_scales;   // per-tensor / per-channel scales
    const void *zero_points;     // same count as the scales, pool element type; may be null
    uint32_t head_dim;
    uint32_t quant_channels;     // per-channel table entries (modes 2, 3)
    // Quantize-on-scatter (op ScatterQuant, single pool): source element type
    // (0 f16, 1 bf16, 2 f32), asymmetric (uint8 pool with zero points), and the
    // per-slot parameters it writes.
    uint32_t qs_src;
    bool qs_asym;
    // one 64-thread workgroup per slot (rows_per_unit 1), else four waves
    // per workgroup with a row each
    bool qs_wave_groups;
    float *qs_scales;
    uint8_t *qs_zero_points;
    // Gated move: the two verdict words an enqueued validation left on the
    // device (smallest failing key, all ones if none; token sum). The copy
    // kernel writes nothing unless the key is all ones and the sum equals
    // gate_tokens. Null: not gated.
    const unsigned long long *gate;
    uint64_t gate_tokens;
};

// Bytes of one page a page-copy workgroup copies, and whether those
// workgroups take chunks in XCD order (4 KiB in dispatch order measured
// fastest: see copy_pages_kernel).
#ifndef HP_PAGE_CHUNK_BYTES
#define HP_PAGE_CHUNK_BYTES 4096
#endif
#ifndef HP_PAGE_XCD
#define HP_PAGE_XCD 0
#endif
constexpr uint32_t kPageChunkBytes = HP_PAGE_CHUNK_BYTES;

// Copy-on-write page copy over `count` pools that share the page IDs.
struct PageCopyJob {
    bool idx64;
    uint32_t vec_bytes;
    uint32_t page_size;
    uint64_t page_bytes;      // P * R
    uint64_t copies;          // entries of src_pages / dst_pages
    const void *src_pages, *dst_pages;
    uint32_t count;
    void *const *pools;
    float *const *scales;     // per pool, may be null (or hold nulls)
};

// Page-range check of a copy's page IDs (checked mode): first failing copy
// index in the workspace head, like the validator.
struct PageCheckJob {
    bool idx64;
    uint64_t copies, num_pages;
    const void *src_pages, *dst_pages;
    void *workspace;
};

struct ValidateJob {
    bool idx64;
    uint64_t num_pages, page_size, num_seqs, num_block_entries;
    const void *block_table, *seq_ptr, *seq_lens, *seq_start;
    void *workspace; // >= 16 bytes: [0] min key, [1] token sum
    // Where the two words go when one workgroup does the whole check
    // (descriptors of at most kValidateOneItems items): device-visible
    // pinned host memory, or null for the workspace.
    void *result;
};
constexpr uint64_t kValidateOneItems = 1 << 16;

// Write-disjointness of a scatter, on a descriptor that passed validation.
// Workspace: [kDisjointAnswer, +8) the smallest clashing sequence (all ones
// when none), then from kDisjointBitmaps two bitmaps of num_pages * page_size
// bits (32-bit words).
struct DisjointJob {
    bool idx64, zero_tail;
    uint64_t num_pages, page_size, num_seqs;
    const void *block_table, *seq_ptr, *seq_lens, *seq_start;
    void *workspace;
};
constexpr uint64_t kDisjointAnswer = 256;
constexpr uint64_t kDisjointBitmaps = 512;
inline uint64_t disjoint_words(uint64_t num_pages, uint64_t page_size) {
    return (num_pages * page_size + 31) / 32;
}
inline uint64_t disjoint_workspace_bytes(uint64_t num_pages, uint64_t page_size) {
    return kDisjointBitmaps + 8 * disjoint_words(num_pages, page_size);
}
// True when launch_validate writes the words to job.result itself.
inline bool validate_writes_result(const ValidateJob &job) {
    const uint64_t n = job.num_block_entries > job.num_seqs + 1 ? job.num_block_entries
                                                                 : job.num_seqs + 1;
    return job.result && n <= kValidateOneItems;
}

// Decode attention over a block-paged K/V cache (hp_attention.hip; its
// launch-shape constants live there).

struct AttentionShape {
    uint32_t heads_per_group;  // kv heads of one workgroup
    uint32_t token_lanes;      // lane groups per head (spare lanes take other tokens)
    uint32_t head_groups;      // grid rows
    uint32_t unit_pages, unit_tokens;
    uint64_t cap_units;        // grid columns: units of the largest batch with total_tokens
    // Shared-prefix pass (cached loads on the matrix-core path): pages of one
    // shared chunk, sequences per row block, the least shared pages of a run,
    // and the most work items the pass can have.
    bool shared;
    uint32_t chunk_pages, seqs_per_block, min_pages;
    uint64_t cap_work;
};

struct AttentionJob {
    bool idx64, bf16, stream_loads;
    bool q8;       // int8 pools with per-slot scales (bf16 queries)
    bool planned;  // the workspace already holds this call's plan (launch_attention_plan)
    uint32_t num_seqs, page_size, num_kv_heads, num_q_heads, head_dim;
    uint64_t total_tokens;
    const void *k_pool, *v_pool, *q;
    const float *k_scales, *v_scales;  // q8 only: N * P each
    const void *block_table, *seq_ptr, *seq_lens;
    float *out;
    float scale;
    void *workspace;  // attention_workspace_bytes(...)
};

// Launch shape of an attention call (q8: int8 pools).
AttentionShape attention_shape(uint64_t num_seqs, uint64_t total_tokens, uint32_t page_size,
                               uint32_t num_kv_heads, uint32_t head_dim, uint32_t num_q_heads,
                               bool stream_loads, bool q8);
// The workspace covers the launch shape with and without streaming loads
// (the streaming hint can choose the kernel), for 16-bit and int8 pools.
uint64_t attention_workspace_bytes(uint64_t num_seqs, uint64_t total_tokens, uint32_t page_size,
                                   uint32_t num_kv_heads, uint32_t head_dim, uint32_t num_q_heads);
hipError_t launch_attention(const AttentionJob &job, hipStream_t stream);
// The planning kernels of launch_attention alone (none for some shapes).
hipError_t launch_attention_plan(const AttentionJob &job, hipStream_t stream);

// Workspace bytes of the plan path: per-sequence offsets and chunk totals.
uint64_t plan_workspace_bytes(uint64_t num_seqs);
// Whether a move over num_seqs sequences may take the plan path by choice.
constexpr bool plan_preferred(Op op, uint64_t num_seqs) {
    return num_seqs >= kPlanMinSeqs && ((HP_PLAN_OPS >> static_cast<int>(op)) & 1);
}

hipError_t launch_copy(const CopyJob &job, hipStream_t stream);
hipError_t launch_validate(const ValidateJob &job, hipStream_t stream);
hipError_t launch_disjoint(const DisjointJob &job, hipStream_t stream);
hipError_t launch_copy_pages(const PageCopyJob &job, hipStream_t stream);
hipError_t launch_check_pages(const PageCheckJob &job, hipStream_t stream);

// Key layout of the validator's atomicMin: check rank in the top byte,
// failing index below it.
constexpr int kKeyShift = 56;
enum CheckRank : uint64_t {
    kRankSeqPtrFirst = 1,
    kRankSeqPtrLast = 2,
    kRankSeqPtrOrder = 3,
    kRankPageRange = 4,
    kRankSeqLen = 5,
};

} // namespace hp
