/*
 * oracle.h -- plain CPU oracle for the block-paged KV layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. It shares no
 * code, header, table or constant with the GPU library and must never be used
 * as a fallback for it.
 *
 * Pages cited (by title and section):
 *   [Hurray] "Block-Paged Layout -- Hurray Format Specification"
 *   [Rust20] "Keep token order across cache pages" (practical LLM in Rust, ch. 20)
 *   [Day51]  "Visualize PagedAttention block layout"
 *
 * Every index array (block_table, seq_ptr, seq_lens, seq_start) is passed as
 * uint64 here; narrowing a uint32 table to this type is lossless, so the index
 * type of a descriptor does not change what the oracle computes.
 *
 * All functions are single-threaded element loops. None allocates memory that
 * outlives the call.
 */
#ifndef BTG_ORACLE_H
#define BTG_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Outcome of oracle_validate, in the order the checks are taken. The numbers
 * are the oracle's own; the test suite maps them to the GPU library's codes. */
enum oracle_check {
    ORACLE_VALID = 0,
    ORACLE_BAD_RANK = 1,        /* [Hurray] Description: rank must be 3 */
    ORACLE_BAD_PAGED_AXIS = 2,  /* [Hurray] Storage Invariants (6) */
    ORACLE_SEQ_PTR_FIRST = 3,   /* (1) seq_ptr[0] = 0 */
    ORACLE_SEQ_PTR_LAST = 4,    /* (1) seq_ptr[num_seqs] = total_logical_pages */
    ORACLE_SEQ_PTR_ORDER = 5,   /* (2) non-decreasing */
    ORACLE_PAGE_RANGE = 6,      /* (3) 0 <= block_table[k] < num_pages */
    ORACLE_SEQ_LEN = 7,         /* token count fits the slice (Partial trailing page) */
    ORACLE_TOTAL_TOKENS = 8     /* total_tokens = sum of counts (Logical Shape) */
};

/* [Hurray] Element Lookup, with the four axis strides of the physical array
 * made explicit so that the same function also evaluates [Rust20]'s
 * [N,B,H_kv,P,d] tutorial layout. Returns the flat element index. */
uint64_t oracle_element_index(const uint64_t *block_table, const uint64_t *seq_ptr,
                              uint64_t s, uint64_t t, uint64_t h, uint64_t d,
                              uint64_t page_size, uint64_t stride_page,
                              uint64_t stride_slot, uint64_t stride_head,
                              uint64_t stride_dim);

/* [Hurray] Storage Invariants (1)-(3), (6), Description (rank 3), plus the two
 * checks the Partial-trailing-page and Logical-Shape paragraphs imply. Returns
 * the first failing check (enum oracle_check) and writes its smallest failing
 * index to *index_out. seq_start may be NULL (every sequence starts at 0). */
int oracle_validate(uint32_t rank, uint32_t paged_axis, uint64_t num_pages,
                    uint64_t page_size, const uint64_t *block_table,
                    uint64_t num_block_entries, const uint64_t *seq_ptr,
                    uint64_t num_seqs, const uint64_t *seq_lens,
                    const uint64_t *seq_start, uint64_t total_tokens,
                    uint64_t *index_out);

/* Whether a scatter's writes land in distinct slots ([Hurray] Prefix Sharing:
 * slices may name the same page, so two written rows, or a row and a zeroed
 * tail slot, can share a slot; a scatter is defined only when they do not).
 * The written slots of sequence s are those of tokens seq_start[s] ..
 * seq_start[s] + seq_lens[s] - 1 and, with zero_tail and seq_lens[s] > 0, the
 * slots after the last of them in its page ([Hurray] Partial trailing page).
 * Returns 1 and writes to *first_out the smallest s one of whose written
 * slots is written more than once (by any sequence, itself included), or
 * returns 0 when every written slot is written once. The descriptor must
 * pass oracle_validate with the same seq_start. seq_start may be NULL. */
int oracle_disjoint_writes(uint64_t num_pages, uint64_t page_size,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           uint64_t num_seqs, const uint64_t *seq_lens,
                           const uint64_t *seq_start, int zero_tail,
                           uint64_t *first_out);

/* Gather: the logical [total_tokens, H, D] tensor, sequences concatenated in
 * index order, token t of sequence s at row (sum of earlier counts) + t.
 * A bit copy of elem_bytes per element. If slot_read_mark is not NULL it has
 * num_pages*page_size bytes and each pool slot the gather reads is set to 1. */
void oracle_gather(const void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                   uint64_t num_heads, uint64_t head_dim,
                   const uint64_t *block_table, const uint64_t *seq_ptr,
                   const uint64_t *seq_lens, uint64_t num_seqs, void *out,
                   uint8_t *slot_read_mark);

/* Gather of selected logical rows only: rows[i] is a row of the logical
 * tensor; out receives rows_count rows of H*D elements. Rows past the total
 * are left untouched and counted in the return value. */
uint64_t oracle_gather_rows(const void *page_pool, uint64_t elem_bytes,
                            uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                            const uint64_t *block_table, const uint64_t *seq_ptr,
                            const uint64_t *seq_lens, uint64_t num_seqs,
                            const uint64_t *rows, uint64_t rows_count, void *out);

/* Scatter: for each sequence s the new tokens occupy logical positions
 * [start_s, start_s + L_s) (start_s = 0 when seq_start is NULL); row i of src
 * belonging to s is written to the pool slot of position start_s + i.
 * With zero_tail != 0, every element of the slots after the last written
 * position, up to the end of that page, is set to zero bytes. */
void oracle_scatter(void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                    uint64_t num_heads, uint64_t head_dim,
                    const uint64_t *block_table, const uint64_t *seq_ptr,
                    const uint64_t *seq_lens, const uint64_t *seq_start,
                    uint64_t num_seqs, const void *src, int zero_tail);

/* fp32 -> bf16, round to nearest, ties to even, on the binary32 bit pattern
 * (IEEE 754 roundTiesToEven). NaN stays NaN (quieted). */
uint16_t oracle_bf16_rne(float x);

/* oracle_bf16_rne applied to n values, one by one. */
void oracle_bf16_rne_array(const float *x, uint64_t n, uint16_t *out);

/* Dequant-gather: out = bf16(fp32(q * scale)) with q the int8 pool element
 * and scale = scales[phys_page * page_size + offset_in_page]
 * ([Hurray] Element Lookup, Per-page-slot parameters). */
void oracle_gather_dequant(const int8_t *page_pool, const float *scales,
                           uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           const uint64_t *seq_lens, uint64_t num_seqs,
                           uint16_t *out);

/* Same arithmetic as oracle_gather_dequant for selected logical rows. */
uint64_t oracle_gather_dequant_rows(const int8_t *page_pool, const float *scales,
                                    uint64_t page_size, uint64_t num_heads,
                                    uint64_t head_dim, const uint64_t *block_table,
                                    const uint64_t *seq_ptr, const uint64_t *seq_lens,
                                    uint64_t num_seqs, const uint64_t *rows,
                                    uint64_t rows_count, uint16_t *out);

/* Quantization schemes ([Hurray] Quantization Compatibility, Per-scheme
 * composition; the scheme tags are the spec's):
 *   0x01 per-tensor        one scale (and zero point) for the whole tensor
 *   0x02 per-channel       axis 1: one per head; axis 2: one per head_dim index
 *   0x03 per-block-affine  axis 0 with block_size == page_size: one per page
 *                          slot, scales[phys * page_size + offset] */
enum oracle_scheme {
    ORACLE_PER_TENSOR = 0x01,
    ORACLE_PER_CHANNEL = 0x02,
    ORACLE_PER_BLOCK_AFFINE = 0x03
};

/* Whether a reader accepts the scheme on a block-paged tensor ([Hurray]
 * Per-scheme composition: per-block-affine needs axis 0 and block_size ==
 * page_size; per-channel composes on axis 1 or 2, axis 0 is forbidden).
 * Returns 1 if accepted, 0 if it must be rejected. */
int oracle_quant_accepts(uint32_t scheme, uint32_t axis, uint64_t block_size,
                         uint64_t page_size);

/* Dequant-gather under any accepted scheme: for every logical element,
 *   out = bf16( fp32(q - zp) * scale )
 * with q the pool element (int8 if q_signed, else uint8), zp the zero point
 * of the same parameter position (0 when zero_points is NULL; same element
 * type as the pool), q - zp exact in integers, one IEEE binary32 multiply and
 * one round to nearest even into bf16 ([Hurray] Element Lookup: dequantize
 * with the scale and zero point of the active scheme). */
void oracle_gather_dequant_scheme(const void *page_pool, int q_signed, uint32_t scheme,
                                  uint32_t axis, const float *scales, const void *zero_points,
                                  uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                                  const uint64_t *block_table, const uint64_t *seq_ptr,
                                  const uint64_t *seq_lens, uint64_t num_seqs, uint16_t *out);

/* Copy-on-write page copy ([Day51] "Copy-on-write for beam search and prefix
 * sharing": a shared block is copied before one request modifies it;
 * [Hurray] Per-page-slot parameters: a page carries its own scales). For
 * i = 0 .. count-1 in order, every element of page src_pages[i] is copied to
 * page dst_pages[i], and, when scales is not NULL, so are that page's
 * page_size slot scales. */
void oracle_copy_pages(void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                       uint64_t num_heads, uint64_t head_dim, float *scales,
                       const uint64_t *src_pages, const uint64_t *dst_pages,
                       uint64_t count);

/* Element types of the attention oracle's inputs (IEEE binary16, bfloat16 =
 * the high half of a binary32, binary32). */
enum oracle_float_type {
    ORACLE_F16 = 3,
    ORACLE_BF16 = 4,
    ORACLE_F32 = 5
};

/* Exact binary64 values of n stored elements of the given type (NaN stays
 * NaN, infinities and subnormals are kept). */
void oracle_decode(uint32_t elem_type, const void *src, uint64_t n, double *out);

/* Decode attention over a block-paged K/V cache ([Day51] "How the attention
 * kernel uses the block table": for each head the kernel walks the sequence's
 * blocks through the table; [Rust20] "Keep token order across cache pages":
 * paging changes only where rows are stored, not the dot products or the
 * weighted sums). For sequence s and query head hq, with kv head
 * hkv = hq / (num_q_heads / num_kv_heads) and the L = seq_lens[s] cached
 * tokens t read through the table ([Hurray] Element Lookup):
 *   x_t = scale * sum_d q[s][hq][d] * K[t][hkv][d]
 *   w_t = exp(x_t - max_t x_t)
 *   out[s][hq][d] = sum_t w_t * V[t][hkv][d] / sum_t w_t
 * all in binary64 from the exact input values. A sequence with no tokens
 * gives zeros. q is [num_seqs, num_q_heads, head_dim]; k_pool and v_pool are
 * [num_pages, page_size, num_kv_heads, head_dim], all of elem_type; out is
 * [num_seqs, num_q_heads, head_dim]. Returns 0, or -1 when num_q_heads is not
 * a multiple of num_kv_heads or a size is zero. */
int oracle_paged_attention(const void *q, const void *k_pool, const void *v_pool,
                           uint32_t elem_type, uint64_t page_size, uint64_t num_kv_heads,
                           uint64_t head_dim, uint64_t num_q_heads, double scale,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           const uint64_t *seq_lens, uint64_t num_seqs, double *out);

/* The same attention over int8 K and V pools with one binary32 scale per
 * physical slot ([Hurray] Per-page-slot parameters: the value of every
 * element of slot page * page_size + r is its code times scales[that slot]):
 * K[t][hkv][d] = k_pool[...] * k_scales[slot of t], likewise V, both exact in
 * binary64; q holds bfloat16 bit patterns. Returns -1 for the cases above or
 * a NULL scale array. */
int oracle_paged_attention_q8(const void *q, const int8_t *k_pool, const float *k_scales,
                              const int8_t *v_pool, const float *v_scales, uint64_t page_size,
                              uint64_t num_kv_heads, uint64_t head_dim, uint64_t num_q_heads,
                              double scale, const uint64_t *block_table,
                              const uint64_t *seq_ptr, const uint64_t *seq_lens,
                              uint64_t num_seqs, double *out);

/* Quantization of one slot's row on write (quantize-on-scatter). The pages
 * fix only where the parameters live ([Hurray] Per-page-slot parameters: one
 * scale, and one zero point for an asymmetric scheme, per physical slot); the
 * scheme document with the formulas is not among them. Reading, with every
 * step one binary32 operation rounded to nearest even:
 *   symmetric int8 (asym = 0): amax = max |x|; scale = amax / 127;
 *     q = clamp(rint(x / scale), -127, 127); amax = 0 gives scale 0, q 0.
 *   asymmetric uint8 (asym = 1): lo = min(0, min x), hi = max(0, max x);
 *     scale = (hi - lo) / 255; z = clamp(rint(-lo / scale), 0, 255);
 *     q = clamp(rint(x / scale) + z, 0, 255); hi = lo gives scale 0, z 0, q 0.
 * x: n binary32 values; q: n int8 (symmetric) or uint8 (asymmetric) codes. */
void oracle_quantize_row(const float *x, uint64_t n, int asym, void *q, float *scale,
                         uint8_t *zero_point);

/* Quantize-on-scatter: oracle_scatter's element placement, with each new
 * token's row (num_heads * head_dim values of src_type ORACLE_F16 / BF16 /
 * F32, converted exactly to binary32) quantized by oracle_quantize_row; the
 * codes go to the pool, the scale to scales[phys * page_size + slot] and, when
 * zero_points is not NULL (asymmetric, uint8 pool), the zero point likewise.
 * With zero_tail the slots of the last written page past the final position
 * get zero codes, scale 0 and zero point 0. */
void oracle_scatter_quant(void *page_pool, float *scales, uint8_t *zero_points,
                          const void *src, uint32_t src_type, uint64_t page_size,
                          uint64_t num_heads, uint64_t head_dim, const uint64_t *block_table,
                          const uint64_t *seq_ptr, const uint64_t *seq_lens,
                          const uint64_t *seq_start, uint64_t num_seqs, int zero_tail);

/* [Rust20] "Count live rows and two kinds of unused payload": buffer-length
 * payload of one layer's K and V arrays. out[] receives, in order:
 *  0 reserved pages      1 active pages
 *  2 allocated slots     3 live slots      4 unused slots
 *  5 tail slots          6 inactive-page slots
 *  7..11 the same five slot counts times elem_bytes
 *  12 contiguous slots for the same capacity (U * capacity)
 * Returns 0, or -1 if length > capacity or a zero size is given. */
int oracle_payload(uint64_t capacity, uint64_t page_tokens, uint64_t length,
                   uint64_t batch, uint64_t kv_heads, uint64_t width,
                   uint64_t elem_bytes, uint64_t out[13]);

#ifdef __cplusplus
}
#endif
#endif
