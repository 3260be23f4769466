/*
 * oracle.c -- plain CPU oracle for the block-paged KV layout.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. It shares no
 * code with the GPU library.
 *
 * Each function is the definition written out one element at a time, in the
 * order the pages state it: no blocking, no fusion, no reordering. Built with
 * gcc -O2 -fno-fast-math -ffp-contract=off; the one floating-point step
 * (dequantisation) is an exact product rounded once to binary32, then once to
 * bf16.
 *
 * Pages cited (by title and section):
 *   [Hurray] "Block-Paged Layout -- Hurray Format Specification"
 *   [Rust20] "Keep token order across cache pages"
 *   [Day51]  "Visualize PagedAttention block layout"
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* [Hurray] Element Lookup:
 *   page_in_seq    = t / page_size
 *   offset_in_page = t mod page_size
 *   phys_page      = block_table[seq_ptr[s] + page_in_seq]
 * and the flat index is the row-major position of (phys_page, offset_in_page,
 * h, d). With strides (P*H*D, H*D, D, 1) this is the page's
 * ((phys_page*page_size + offset_in_page)*num_heads + h)*head_dim + d; with
 * [Rust20] "Include the batch, shared head and feature" strides
 * (B*H*P*d, d, P*d, 1) it is that tutorial's [N,B,H_kv,P,d] index at lane 0. */
uint64_t oracle_element_index(const uint64_t *block_table, const uint64_t *seq_ptr,
                              uint64_t s, uint64_t t, uint64_t h, uint64_t d,
                              uint64_t page_size, uint64_t stride_page,
                              uint64_t stride_slot, uint64_t stride_head,
                              uint64_t stride_dim)
{
    uint64_t page_in_seq = t / page_size;
    uint64_t offset_in_page = t % page_size;
    uint64_t phys_page = block_table[seq_ptr[s] + page_in_seq];
    return phys_page * stride_page + offset_in_page * stride_slot +
           h * stride_head + d * stride_dim;
}

/* The interchange layout [num_pages, page_size, num_heads, head_dim]
 * ([Hurray] Element Lookup; Framework Compliance). */
static uint64_t pool_index(const uint64_t *block_table, const uint64_t *seq_ptr,
                           uint64_t s, uint64_t t, uint64_t h, uint64_t d,
                           uint64_t P, uint64_t H, uint64_t D)
{
    return oracle_element_index(block_table, seq_ptr, s, t, h, d, P, P * H * D,
                                H * D, D, 1);
}

/* [Hurray] Description (rank 3 only), Storage Invariants (1), (2), (3), (6),
 * Partial trailing page (a count may not run past its slice) and Logical
 * Shape (total_tokens is the sum of the counts). The first failing check in
 * that order is returned, with the smallest index at which it fails. */
int oracle_validate(uint32_t rank, uint32_t paged_axis, uint64_t num_pages,
                    uint64_t page_size, const uint64_t *block_table,
                    uint64_t num_block_entries, const uint64_t *seq_ptr,
                    uint64_t num_seqs, const uint64_t *seq_lens,
                    const uint64_t *seq_start, uint64_t total_tokens,
                    uint64_t *index_out)
{
    uint64_t s, k;
    unsigned __int128 sum = 0;

    *index_out = 0;
    if (rank != 3)
        return ORACLE_BAD_RANK;
    if (paged_axis != 0)
        return ORACLE_BAD_PAGED_AXIS;
    /* (1) seq_ptr[0] = 0 and seq_ptr[num_seqs] = total_logical_pages, the
     * latter being the number of entries the block_table buffer holds. */
    if (seq_ptr[0] != 0)
        return ORACLE_SEQ_PTR_FIRST;
    if (seq_ptr[num_seqs] != num_block_entries) {
        *index_out = num_seqs;
        return ORACLE_SEQ_PTR_LAST;
    }
    /* (2) seq_ptr[s] <= seq_ptr[s+1] for all s. */
    for (s = 0; s < num_seqs; s++) {
        if (seq_ptr[s] > seq_ptr[s + 1]) {
            *index_out = s;
            return ORACLE_SEQ_PTR_ORDER;
        }
    }
    /* (3) 0 <= block_table[k] < num_pages (unsigned, so only the upper bound). */
    for (k = 0; k < num_block_entries; k++) {
        if (block_table[k] >= num_pages) {
            *index_out = k;
            return ORACLE_PAGE_RANGE;
        }
    }
    /* The last position a sequence touches must lie in a page of its slice. */
    for (s = 0; s < num_seqs; s++) {
        unsigned __int128 slots =
            (unsigned __int128)(seq_ptr[s + 1] - seq_ptr[s]) * page_size;
        unsigned __int128 end = (unsigned __int128)seq_lens[s] +
                                (seq_start ? seq_start[s] : 0);
        if (end > slots) {
            *index_out = s;
            return ORACLE_SEQ_LEN;
        }
    }
    /* [Hurray] Logical Shape: the logical tensor's first extent counts every
     * sequence's tokens, so the counts must add up to total_tokens. */
    for (s = 0; s < num_seqs; s++)
        sum += seq_lens[s];
    if (sum != (unsigned __int128)total_tokens)
        return ORACLE_TOTAL_TOKENS;
    return ORACLE_VALID;
}

/* Visits the slots sequence s writes in a scatter: its tokens' slots, then,
 * with zero_tail, the slots after the last token in that token's page. */
static void written_slots(uint64_t page_size, const uint64_t *block_table,
                          const uint64_t *seq_ptr, const uint64_t *seq_lens,
                          const uint64_t *seq_start, int zero_tail, uint64_t s,
                          void (*visit)(uint64_t slot, void *ctx), void *ctx)
{
    uint64_t start = seq_start ? seq_start[s] : 0;
    uint64_t t, r;
    for (t = start; t < start + seq_lens[s]; t++)
        visit(block_table[seq_ptr[s] + t / page_size] * page_size + t % page_size, ctx);
    if (zero_tail && seq_lens[s] > 0) {
        uint64_t last = start + seq_lens[s] - 1;
        uint64_t page = block_table[seq_ptr[s] + last / page_size];
        for (r = last % page_size + 1; r < page_size; r++)
            visit(page * page_size + r, ctx);
    }
}

static void count_write(uint64_t slot, void *ctx)
{
    unsigned char *count = (unsigned char *)ctx;
    if (count[slot] < 2)
        count[slot]++;
}

struct shared_probe {
    const unsigned char *count;
    int hit;
};

static void probe_write(uint64_t slot, void *ctx)
{
    struct shared_probe *p = (struct shared_probe *)ctx;
    if (p->count[slot] >= 2)
        p->hit = 1;
}

/* [Hurray] Prefix Sharing and Partial trailing page: count the writes of
 * every slot over all sequences, then find the first sequence that writes a
 * slot counted twice. */
int oracle_disjoint_writes(uint64_t num_pages, uint64_t page_size,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           uint64_t num_seqs, const uint64_t *seq_lens,
                           const uint64_t *seq_start, int zero_tail,
                           uint64_t *first_out)
{
    unsigned char *count = (unsigned char *)calloc(num_pages * page_size + 1, 1);
    uint64_t s;
    int found = 0;

    *first_out = 0;
    if (!count)
        abort();
    for (s = 0; s < num_seqs; s++)
        written_slots(page_size, block_table, seq_ptr, seq_lens, seq_start, zero_tail, s,
                      count_write, count);
    for (s = 0; s < num_seqs && !found; s++) {
        struct shared_probe p = {count, 0};
        written_slots(page_size, block_table, seq_ptr, seq_lens, seq_start, zero_tail, s,
                      probe_write, &p);
        if (p.hit) {
            *first_out = s;
            found = 1;
        }
    }
    free(count);
    return found;
}

/* Gather in logical order: sequence by sequence, token by token, head by
 * head, dimension by dimension ([Hurray] Logical Shape, Element Lookup). Only
 * tokens t < L_s are visited, so no slot past a sequence's count is read
 * ([Hurray] Partial trailing page). */
void oracle_gather(const void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                   uint64_t num_heads, uint64_t head_dim,
                   const uint64_t *block_table, const uint64_t *seq_ptr,
                   const uint64_t *seq_lens, uint64_t num_seqs, void *out,
                   uint8_t *slot_read_mark)
{
    const unsigned char *pool = (const unsigned char *)page_pool;
    unsigned char *dst = (unsigned char *)out;
    uint64_t row = 0;
    uint64_t s, t, h, d;

    for (s = 0; s < num_seqs; s++) {
        for (t = 0; t < seq_lens[s]; t++) {
            for (h = 0; h < num_heads; h++) {
                for (d = 0; d < head_dim; d++) {
                    uint64_t src = pool_index(block_table, seq_ptr, s, t, h, d,
                                              page_size, num_heads, head_dim);
                    uint64_t o = (row * num_heads + h) * head_dim + d;
                    memcpy(dst + o * elem_bytes, pool + src * elem_bytes, elem_bytes);
                    if (slot_read_mark)
                        slot_read_mark[src / (num_heads * head_dim)] = 1;
                }
            }
            row++;
        }
    }
}

/* Find the sequence and in-sequence position of logical row `row`, walking
 * the counts in order ([Hurray] Logical Shape). Returns 0 if past the end. */
static int locate_row(const uint64_t *seq_lens, uint64_t num_seqs, uint64_t row,
                      uint64_t *s_out, uint64_t *t_out)
{
    uint64_t s, first = 0;
    for (s = 0; s < num_seqs; s++) {
        if (row < first + seq_lens[s]) {
            *s_out = s;
            *t_out = row - first;
            return 1;
        }
        first += seq_lens[s];
    }
    return 0;
}

uint64_t oracle_gather_rows(const void *page_pool, uint64_t elem_bytes,
                            uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                            const uint64_t *block_table, const uint64_t *seq_ptr,
                            const uint64_t *seq_lens, uint64_t num_seqs,
                            const uint64_t *rows, uint64_t rows_count, void *out)
{
    const unsigned char *pool = (const unsigned char *)page_pool;
    unsigned char *dst = (unsigned char *)out;
    uint64_t i, h, d, missing = 0;

    for (i = 0; i < rows_count; i++) {
        uint64_t s, t;
        if (!locate_row(seq_lens, num_seqs, rows[i], &s, &t)) {
            missing++;
            continue;
        }
        for (h = 0; h < num_heads; h++) {
            for (d = 0; d < head_dim; d++) {
                uint64_t src = pool_index(block_table, seq_ptr, s, t, h, d,
                                          page_size, num_heads, head_dim);
                uint64_t o = (i * num_heads + h) * head_dim + d;
                memcpy(dst + o * elem_bytes, pool + src * elem_bytes, elem_bytes);
            }
        }
    }
    return missing;
}

/* Scatter: the inverse element move. New token i of sequence s sits at
 * logical position start_s + i and is stored through the same lookup
 * ([Hurray] Element Lookup). With zero_tail the slots of the last written
 * page past the final position are cleared ([Hurray] Partial trailing page:
 * a writer should zero the unused slots). */
void oracle_scatter(void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                    uint64_t num_heads, uint64_t head_dim,
                    const uint64_t *block_table, const uint64_t *seq_ptr,
                    const uint64_t *seq_lens, const uint64_t *seq_start,
                    uint64_t num_seqs, const void *src, int zero_tail)
{
    unsigned char *pool = (unsigned char *)page_pool;
    const unsigned char *in = (const unsigned char *)src;
    uint64_t row = 0;
    uint64_t s, i, h, d;

    for (s = 0; s < num_seqs; s++) {
        uint64_t start = seq_start ? seq_start[s] : 0;
        for (i = 0; i < seq_lens[s]; i++) {
            uint64_t t = start + i;
            for (h = 0; h < num_heads; h++) {
                for (d = 0; d < head_dim; d++) {
                    uint64_t dst = pool_index(block_table, seq_ptr, s, t, h, d,
                                              page_size, num_heads, head_dim);
                    uint64_t o = (row * num_heads + h) * head_dim + d;
                    memcpy(pool + dst * elem_bytes, in + o * elem_bytes, elem_bytes);
                }
            }
            row++;
        }
        if (zero_tail && seq_lens[s] > 0) {
            uint64_t end = start + seq_lens[s];
            uint64_t t;
            /* Positions end .. (end rounded up to a page) share the last
             * written page; none of them holds a valid token. */
            for (t = end; t % page_size != 0; t++) {
                for (h = 0; h < num_heads; h++) {
                    for (d = 0; d < head_dim; d++) {
                        uint64_t dst = pool_index(block_table, seq_ptr, s, t, h, d,
                                                  page_size, num_heads, head_dim);
                        memset(pool + dst * elem_bytes, 0, elem_bytes);
                    }
                }
            }
        }
    }
}

/* IEEE 754 roundTiesToEven from binary32 to the bfloat16 format (binary32's
 * sign, exponent and top 7 fraction bits). The 16 discarded bits are compared
 * with the halfway value 0x8000; above it, or equal with an odd kept part,
 * the kept part is incremented (a carry into the exponent gives the next
 * binade or infinity, which is the correctly rounded result). NaN is kept as
 * a NaN with the quiet bit set. */
uint16_t oracle_bf16_rne(float x)
{
    uint32_t bits;
    uint32_t kept, dropped;

    memcpy(&bits, &x, sizeof bits);
    if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0)
        return (uint16_t)((bits >> 16) | 0x0040u);
    kept = bits >> 16;
    dropped = bits & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1;
    return (uint16_t)kept;
}

void oracle_bf16_rne_array(const float *x, uint64_t n, uint16_t *out)
{
    uint64_t i;
    for (i = 0; i < n; i++)
        out[i] = oracle_bf16_rne(x[i]);
}

/* One dequantised element: the int8 value times the slot's fp32 scale. The
 * exact product of an 8-bit integer and a 24-bit significand fits binary64,
 * so (float)((double)q * scale) is the product rounded once to binary32, as a
 * single IEEE fp32 multiply gives; then one rounding to bf16. */
static uint16_t dequant_one(int8_t q, float scale)
{
    double exact = (double)q * (double)scale;
    float product = (float)exact;
    return oracle_bf16_rne(product);
}

void oracle_gather_dequant(const int8_t *page_pool, const float *scales,
                           uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           const uint64_t *seq_lens, uint64_t num_seqs,
                           uint16_t *out)
{
    uint64_t row = 0;
    uint64_t s, t, h, d;

    for (s = 0; s < num_seqs; s++) {
        for (t = 0; t < seq_lens[s]; t++) {
            /* [Hurray] Per-page-slot parameters: scales[p * page_size + i]. */
            uint64_t phys = block_table[seq_ptr[s] + t / page_size];
            float scale = scales[phys * page_size + t % page_size];
            for (h = 0; h < num_heads; h++) {
                for (d = 0; d < head_dim; d++) {
                    uint64_t src = pool_index(block_table, seq_ptr, s, t, h, d,
                                              page_size, num_heads, head_dim);
                    out[(row * num_heads + h) * head_dim + d] =
                        dequant_one(page_pool[src], scale);
                }
            }
            row++;
        }
    }
}

uint64_t oracle_gather_dequant_rows(const int8_t *page_pool, const float *scales,
                                    uint64_t page_size, uint64_t num_heads,
                                    uint64_t head_dim, const uint64_t *block_table,
                                    const uint64_t *seq_ptr, const uint64_t *seq_lens,
                                    uint64_t num_seqs, const uint64_t *rows,
                                    uint64_t rows_count, uint16_t *out)
{
    uint64_t i, h, d, missing = 0;

    for (i = 0; i < rows_count; i++) {
        uint64_t s, t, phys;
        float scale;
        if (!locate_row(seq_lens, num_seqs, rows[i], &s, &t)) {
            missing++;
            continue;
        }
        phys = block_table[seq_ptr[s] + t / page_size];
        scale = scales[phys * page_size + t % page_size];
        for (h = 0; h < num_heads; h++) {
            for (d = 0; d < head_dim; d++) {
                uint64_t src = pool_index(block_table, seq_ptr, s, t, h, d,
                                          page_size, num_heads, head_dim);
                out[(i * num_heads + h) * head_dim + d] =
                    dequant_one(page_pool[src], scale);
            }
        }
    }
    return missing;
}

int oracle_quant_accepts(uint32_t scheme, uint32_t axis, uint64_t block_size,
                         uint64_t page_size)
{
    if (scheme == ORACLE_PER_TENSOR)
        return 1;
    if (scheme == ORACLE_PER_CHANNEL)
        return axis == 1 || axis == 2;
    if (scheme == ORACLE_PER_BLOCK_AFFINE)
        return axis == 0 && block_size == page_size;
    return 0;
}

void oracle_gather_dequant_scheme(const void *page_pool, int q_signed, uint32_t scheme,
                                  uint32_t axis, const float *scales, const void *zero_points,
                                  uint64_t page_size, uint64_t num_heads, uint64_t head_dim,
                                  const uint64_t *block_table, const uint64_t *seq_ptr,
                                  const uint64_t *seq_lens, uint64_t num_seqs, uint16_t *out)
{
    const int8_t *qs = (const int8_t *)page_pool;
    const uint8_t *qu = (const uint8_t *)page_pool;
    const int8_t *zs = (const int8_t *)zero_points;
    const uint8_t *zu = (const uint8_t *)zero_points;
    uint64_t row = 0;
    uint64_t s, t, h, d;

    for (s = 0; s < num_seqs; s++) {
        for (t = 0; t < seq_lens[s]; t++) {
            uint64_t phys = block_table[seq_ptr[s] + t / page_size];
            for (h = 0; h < num_heads; h++) {
                for (d = 0; d < head_dim; d++) {
                    uint64_t src = pool_index(block_table, seq_ptr, s, t, h, d, page_size,
                                              num_heads, head_dim);
                    /* parameter position of this element under the scheme */
                    uint64_t k = 0;
                    int32_t q, zp = 0;
                    double exact;
                    if (scheme == ORACLE_PER_CHANNEL)
                        k = axis == 1 ? h : d;
                    else if (scheme == ORACLE_PER_BLOCK_AFFINE)
                        k = phys * page_size + t % page_size;
                    q = q_signed ? (int32_t)qs[src] : (int32_t)qu[src];
                    if (zero_points)
                        zp = q_signed ? (int32_t)zs[k] : (int32_t)zu[k];
                    /* q - zp is an exact small integer; times the scale exactly
                     * in binary64, then one rounding to binary32 and one to bf16 */
                    exact = (double)(q - zp) * (double)scales[k];
                    out[(row * num_heads + h) * head_dim + d] = oracle_bf16_rne((float)exact);
                }
            }
            row++;
        }
    }
}

/* Copy-on-write page copy: page by page, slot by slot, element by element,
 * in the order the copies are listed. */
void oracle_copy_pages(void *page_pool, uint64_t elem_bytes, uint64_t page_size,
                       uint64_t num_heads, uint64_t head_dim, float *scales,
                       const uint64_t *src_pages, const uint64_t *dst_pages,
                       uint64_t count)
{
    unsigned char *pool = (unsigned char *)page_pool;
    uint64_t i, slot, h, d;

    for (i = 0; i < count; i++) {
        for (slot = 0; slot < page_size; slot++) {
            for (h = 0; h < num_heads; h++) {
                for (d = 0; d < head_dim; d++) {
                    uint64_t from = ((src_pages[i] * page_size + slot) * num_heads + h) *
                                    head_dim + d;
                    uint64_t to = ((dst_pages[i] * page_size + slot) * num_heads + h) *
                                  head_dim + d;
                    memcpy(pool + to * elem_bytes, pool + from * elem_bytes, elem_bytes);
                }
            }
            if (scales)
                scales[dst_pages[i] * page_size + slot] =
                    scales[src_pages[i] * page_size + slot];
        }
    }
}

/* IEEE 754 binary16: sign bit, 5-bit exponent biased by 15, 10-bit
 * fraction. Exponent 0 holds zero and the subnormals f * 2^-24; exponent 31
 * holds the infinities (f = 0) and NaNs. Otherwise the value is
 * (1024 + f) * 2^(e - 25). */
static double half_value(uint16_t b)
{
    int e = (b >> 10) & 31;
    int f = b & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return (b >> 15) ? -v : v;
}

/* bfloat16 is the upper 16 bits of a binary32. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double element_value(uint32_t elem_type, const void *base, uint64_t i)
{
    if (elem_type == ORACLE_F32) {
        float f;
        memcpy(&f, (const unsigned char *)base + 4 * i, sizeof f);
        return (double)f;
    }
    uint16_t b;
    memcpy(&b, (const unsigned char *)base + 2 * i, sizeof b);
    return elem_type == ORACLE_F16 ? half_value(b) : bf16_value(b);
}

void oracle_decode(uint32_t elem_type, const void *src, uint64_t n, double *out)
{
    uint64_t i;
    for (i = 0; i < n; i++)
        out[i] = element_value(elem_type, src, i);
}

/* A K or V pool as the attention oracle reads it: stored floats of one
 * element type, or (scales != NULL) int8 codes whose value is the code times
 * its slot's scale ([Hurray] Per-page-slot parameters: one scale per
 * physical slot, for every element of the slot's row; the product of an
 * 8-bit code and a binary32 scale is exact in binary64). */
struct kv_pool {
    const void *base;
    uint32_t elem_type;    /* ORACLE_F16 / BF16 / F32 (when scales is NULL) */
    const float *scales;   /* int8 codes: num_pages * page_size scales */
    uint64_t row_elems;    /* elements of one slot: num_kv_heads * head_dim */
};

static double kv_value(const struct kv_pool *p, uint64_t i)
{
    if (p->scales)
        return (double)((const int8_t *)p->base)[i] * (double)p->scales[i / p->row_elems];
    return element_value(p->elem_type, p->base, i);
}

/* Softmax attention of one query row over a sequence's cached tokens, the
 * keys and values found through the block table one token at a time. */
static int attention(const void *q, uint32_t q_type, const struct kv_pool *k,
                     const struct kv_pool *v, uint64_t page_size, uint64_t num_kv_heads,
                     uint64_t head_dim, uint64_t num_q_heads, double scale,
                     const uint64_t *block_table, const uint64_t *seq_ptr,
                     const uint64_t *seq_lens, uint64_t num_seqs, double *out)
{
    uint64_t s, hq, t, d, group, max_len = 0;
    double *x;

    if (!page_size || !num_kv_heads || !head_dim || !num_q_heads ||
        num_q_heads % num_kv_heads)
        return -1;
    group = num_q_heads / num_kv_heads;
    for (s = 0; s < num_seqs; s++)
        if (seq_lens[s] > max_len)
            max_len = seq_lens[s];
    x = (double *)malloc((max_len ? max_len : 1) * sizeof(double));
    if (!x)
        return -1;

    for (s = 0; s < num_seqs; s++) {
        uint64_t L = seq_lens[s];
        for (hq = 0; hq < num_q_heads; hq++) {
            uint64_t hkv = hq / group;
            double *o = out + (s * num_q_heads + hq) * head_dim;
            double m = -INFINITY, denom = 0.0;
            if (L == 0) {
                for (d = 0; d < head_dim; d++)
                    o[d] = 0.0;
                continue;
            }
            /* scores x_t = scale * q . k_t */
            for (t = 0; t < L; t++) {
                double dot = 0.0;
                for (d = 0; d < head_dim; d++) {
                    double qv = element_value(q_type, q, (s * num_q_heads + hq) * head_dim + d);
                    double kv = kv_value(k, pool_index(block_table, seq_ptr, s, t, hkv, d,
                                                       page_size, num_kv_heads, head_dim));
                    dot += qv * kv;
                }
                x[t] = scale * dot;
                if (x[t] > m)
                    m = x[t];
            }
            /* weights relative to the largest score, then the weighted mean */
            for (t = 0; t < L; t++) {
                x[t] = exp(x[t] - m);
                denom += x[t];
            }
            for (d = 0; d < head_dim; d++) {
                double num = 0.0;
                for (t = 0; t < L; t++)
                    num += x[t] * kv_value(v, pool_index(block_table, seq_ptr, s, t, hkv, d,
                                                         page_size, num_kv_heads, head_dim));
                o[d] = num / denom;
            }
        }
    }
    free(x);
    return 0;
}

int oracle_paged_attention(const void *q, const void *k_pool, const void *v_pool,
                           uint32_t elem_type, uint64_t page_size, uint64_t num_kv_heads,
                           uint64_t head_dim, uint64_t num_q_heads, double scale,
                           const uint64_t *block_table, const uint64_t *seq_ptr,
                           const uint64_t *seq_lens, uint64_t num_seqs, double *out)
{
    const struct kv_pool k = {k_pool, elem_type, NULL, num_kv_heads * head_dim};
    const struct kv_pool v = {v_pool, elem_type, NULL, num_kv_heads * head_dim};
    return attention(q, elem_type, &k, &v, page_size, num_kv_heads, head_dim, num_q_heads,
                     scale, block_table, seq_ptr, seq_lens, num_seqs, out);
}

int oracle_paged_attention_q8(const void *q, const int8_t *k_pool, const float *k_scales,
                              const int8_t *v_pool, const float *v_scales, uint64_t page_size,
                              uint64_t num_kv_heads, uint64_t head_dim, uint64_t num_q_heads,
                              double scale, const uint64_t *block_table,
                              const uint64_t *seq_ptr, const uint64_t *seq_lens,
                              uint64_t num_seqs, double *out)
{
    const struct kv_pool k = {k_pool, 0, k_scales, num_kv_heads * head_dim};
    const struct kv_pool v = {v_pool, 0, v_scales, num_kv_heads * head_dim};
    if (!k_scales || !v_scales)
        return -1;
    return attention(q, ORACLE_BF16, &k, &v, page_size, num_kv_heads, head_dim, num_q_heads,
                     scale, block_table, seq_ptr, seq_lens, num_seqs, out);
}

/* One binary32 value as rint would give it, clamped to [lo, hi] (exact: the
 * bounds are integers). */
static float clamp_rint(float v, float lo, float hi)
{
    float r = rintf(v);
    return r < lo ? lo : (r > hi ? hi : r);
}

void oracle_quantize_row(const float *x, uint64_t n, int asym, void *q, float *scale,
                         uint8_t *zero_point)
{
    uint64_t i;
    if (!asym) {
        int8_t *out = (int8_t *)q;
        float amax = 0.0f, sc;
        for (i = 0; i < n; i++) {
            float a = fabsf(x[i]);
            if (a > amax)
                amax = a;
        }
        sc = amax / 127.0f;
        *scale = sc;
        for (i = 0; i < n; i++)
            out[i] = sc == 0.0f ? 0 : (int8_t)clamp_rint(x[i] / sc, -127.0f, 127.0f);
    } else {
        uint8_t *out = (uint8_t *)q;
        float lo = 0.0f, hi = 0.0f, sc, z;
        for (i = 0; i < n; i++) {
            if (x[i] < lo)
                lo = x[i];
            if (x[i] > hi)
                hi = x[i];
        }
        sc = (hi - lo) / 255.0f;
        z = sc == 0.0f ? 0.0f : clamp_rint(-lo / sc, 0.0f, 255.0f);
        *scale = sc;
        *zero_point = (uint8_t)z;
        for (i = 0; i < n; i++) {
            if (sc == 0.0f) {
                out[i] = 0;
            } else {
                float c = rintf(x[i] / sc) + z; /* small integers: exact */
                out[i] = (uint8_t)(c < 0.0f ? 0.0f : (c > 255.0f ? 255.0f : c));
            }
        }
    }
}

void oracle_scatter_quant(void *page_pool, float *scales, uint8_t *zero_points,
                          const void *src, uint32_t src_type, uint64_t page_size,
                          uint64_t num_heads, uint64_t head_dim, const uint64_t *block_table,
                          const uint64_t *seq_ptr, const uint64_t *seq_lens,
                          const uint64_t *seq_start, uint64_t num_seqs, int zero_tail)
{
    unsigned char *pool = (unsigned char *)page_pool;
    const uint64_t n = num_heads * head_dim;
    float *x = (float *)malloc((n ? n : 1) * sizeof(float));
    unsigned char *codes = (unsigned char *)malloc(n ? n : 1);
    uint64_t row = 0;
    uint64_t s, i, h, d, e;

    if (!x || !codes) {
        free(x);
        free(codes);
        return;
    }
    for (s = 0; s < num_seqs; s++) {
        uint64_t start = seq_start ? seq_start[s] : 0;
        for (i = 0; i < seq_lens[s]; i++) {
            uint64_t t = start + i;
            uint64_t phys = block_table[seq_ptr[s] + t / page_size];
            uint64_t slot = phys * page_size + t % page_size;
            float sc;
            uint8_t zp = 0;
            for (e = 0; e < n; e++)
                x[e] = (float)element_value(src_type, src, row * n + e);
            oracle_quantize_row(x, n, zero_points != NULL, codes, &sc, &zp);
            for (h = 0; h < num_heads; h++)
                for (d = 0; d < head_dim; d++)
                    pool[pool_index(block_table, seq_ptr, s, t, h, d, page_size, num_heads,
                                    head_dim)] = codes[h * head_dim + d];
            scales[slot] = sc;
            if (zero_points)
                zero_points[slot] = zp;
            row++;
        }
        if (zero_tail && seq_lens[s] > 0) {
            uint64_t t;
            for (t = start + seq_lens[s]; t % page_size != 0; t++) {
                uint64_t phys = block_table[seq_ptr[s] + t / page_size];
                uint64_t slot = phys * page_size + t % page_size;
                for (h = 0; h < num_heads; h++)
                    for (d = 0; d < head_dim; d++)
                        pool[pool_index(block_table, seq_ptr, s, t, h, d, page_size,
                                        num_heads, head_dim)] = 0;
                scales[slot] = 0.0f;
                if (zero_points)
                    zero_points[slot] = 0;
            }
        }
    }
    free(x);
    free(codes);
}

/* [Rust20] "Count live rows and two kinds of unused payload": with
 * U = 2*B*H_kv*d slots per token position (K and V), A = ceil(n/P) active
 * pages and ceil(C/P)*P reserved positions,
 *   allocated = U * ceil(C/P) * P      live     = U * n
 *   tail      = U * (A*P - n)          inactive = U * (ceil(C/P)*P - A*P)
 *   unused    = allocated - live.
 * "A rounded page can reserve more than contiguous storage": contiguous
 * storage for capacity C holds U*C slots. */
int oracle_payload(uint64_t capacity, uint64_t page_tokens, uint64_t length,
                   uint64_t batch, uint64_t kv_heads, uint64_t width,
                   uint64_t elem_bytes, uint64_t out[13])
{
    uint64_t per_position, reserved_pages, active_pages, reserved_positions;
    uint64_t active_positions, i;

    if (capacity == 0 || page_tokens == 0 || length > capacity)
        return -1;
    per_position = 2 * batch * kv_heads * width;
    reserved_pages = (capacity + page_tokens - 1) / page_tokens;
    active_pages = (length + page_tokens - 1) / page_tokens;
    reserved_positions = reserved_pages * page_tokens;
    active_positions = active_pages * page_tokens;

    out[0] = reserved_pages;
    out[1] = active_pages;
    out[2] = per_position * reserved_positions;
    out[3] = per_position * length;
    out[4] = out[2] - out[3];
    out[5] = per_position * (active_positions - length);
    out[6] = per_position * (reserved_positions - active_positions);
    for (i = 0; i < 5; i++)
        out[7 + i] = out[2 + i] * elem_bytes;
    out[12] = per_position * capacity;
    return 0;
}
