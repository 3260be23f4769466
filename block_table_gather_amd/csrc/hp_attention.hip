// hp_attention.hip -- decode attention that reads K and V through the block
// table, for gfx950.
//
// What is computed ("Visualize PagedAttention block layout", How the attention
// kernel uses the block table; "Keep token order across cache pages": paging
// decides where rows are stored, not what attention computes): for each
// sequence s and query head hq, with kv head h = hq / G (G = Hq / Hkv query
// heads share one kv head),
//   x_t = scale * q[s][hq] . K[t][h],  out[s][hq] = sum_t e^{x_t} V[t][h] / sum_t e^{x_t}
// over the sequence's L_s cached tokens, whose rows are found through the
// block table as in "Block-Paged Layout -- Hurray Format Specification",
// Element Lookup. A sequence with no tokens gives zeros.
//
// Design (HBM-bound: each cached K/V byte is read once; the contraction is a
// dot product per token and head, so it runs on the vector ALUs in fp32):
//  * A sequence is cut into units of U tokens (U a multiple of the page size,
//    chosen on the host so that the grid has one to a few thousand
//    workgroups). Up to kAttnFusedSeqs sequences every workgroup rebuilds the
//    running unit count unit_end[s] in LDS from the token counts and finds
//    its sequence by binary search there; beyond that a plan kernel writes
//    unit_end and the sequence of every unit to the workspace.
//  * Workgroup (unit, head group, query chunk) covers up to 256 / (D / 8) kv
//    heads and up to 8 of each kv head's query heads. D / 8
//    lanes hold one head row (16 bytes each: 8 fp16/bf16 values), so one
//    token's row of those heads is one contiguous read. When the kv heads do
//    not fill the workgroup, the spare lane groups take other tokens of the
//    unit (token lanes) and their softmax states are merged through LDS.
//  * The unit's page IDs are staged in LDS once. Each lane group streams
//    batches of tokens: all K and V loads of a batch are issued before any is
//    used; q . k runs on v_dot2 (two 16-bit products per instruction, fp32
//    accumulation) and is summed across the head's lanes with DPP row
//    operations; an online softmax (running max, base 2) rescales the
//    accumulator once per batch.
//  * With three or more query heads per kv head (two with streaming loads)
//    and head_dim 64 or 128, the matrix-core kernel below takes the call
//    instead; with cached loads its grid also carries the shared-prefix pass.
//  * Each unit writes (max, sum of weights, unnormalised weighted sum of V)
//    per query head to the workspace, and a combine kernel merges a
//    sequence's units and divides. A sequence held by one unit is normalised
//    and written directly by its workgroup, and spare workgroups write the
//    zeros of sequences without tokens. (Merging in the last unit to finish
//    needs an agent-scope release per workgroup, which writes the XCD's L2
//    back; it measured 3x slower than the second launch.)
#include "hp_device.h"
#include "hp_internal.h"

#include <stdint.h>
#include <type_traits>

namespace hp {

// Workgroups aimed at per launch (a unit holds enough pages to reach about
// this many), and the most pages one unit may hold.
#ifndef HP_ATTN_TARGET_GROUPS_MHA
#define HP_ATTN_TARGET_GROUPS_MHA 1024
#endif
// Grouped query heads with cached loads: measured on MI355X, prefix batch
// (shared-prefix pass, three waves per SIMD), G = 4 / 8: 3,072 workgroups
// 94.9 / 109.9 us, 4,096 93.4 / 107.5 us, 5,120 94.9 / 110.0 us, 6,144
// 96.2 / 113.5 us.
#ifndef HP_ATTN_TARGET_GROUPS_GQA
#define HP_ATTN_TARGET_GROUPS_GQA 4096
#endif
constexpr uint64_t kAttnTargetGroupsMha = HP_ATTN_TARGET_GROUPS_MHA;
constexpr uint64_t kAttnTargetGroupsGqa = HP_ATTN_TARGET_GROUPS_GQA;
// Grouped query heads with streaming loads (pages read once) take longer
// units: measured on MI355X, decode batch at G = 4 / 8 (int8 pools at G = 4),
// grid with interleaved head groups, cold caches: 3,072 workgroups 191.6 /
// 206.3 (117.7) us, 2,048 187.6 / 199.4 (113.1) us, 1,536 188.9 / 202.0
// (114.7) us, 1,024 189.4 / 201.6 (116.1) us.
#ifndef HP_ATTN_TARGET_GROUPS_GQA_STREAM
#define HP_ATTN_TARGET_GROUPS_GQA_STREAM 2048
#endif
constexpr uint64_t kAttnTargetGroupsGqaStream = HP_ATTN_TARGET_GROUPS_GQA_STREAM;
constexpr uint64_t kAttnMaxUnitPages = 256;
// Smallest unit, in tokens per query-head slot of a lane group.
#ifndef HP_ATTN_MIN_UNIT_TOKENS_PER_SLOT
#define HP_ATTN_MIN_UNIT_TOKENS_PER_SLOT 8
#endif
constexpr uint64_t kAttnMinUnitTokensPerSlot = HP_ATTN_MIN_UNIT_TOKENS_PER_SLOT;
// Up to this many sequences the attention kernels count units themselves
// (unit table in LDS, 4 bytes per sequence); beyond it a plan kernel runs.
constexpr uint32_t kAttnFusedSeqs = 4096;

namespace {

constexpr uint32_t kAttnThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct F16 {
    static constexpr bool bf16 = false;
};
struct BF16 {
    static constexpr bool bf16 = true;
};

struct AArgs {
    const unsigned char *k_pool, *v_pool, *q;
    const void *block_table, *seq_ptr, *seq_lens;
    const uint32_t *unit_end, *unit_seq;
    float *part_ml;    // [cap_units][Hq][2]: running max (base 2), sum of weights
    float *part_acc;   // [cap_units][Hq][D]: unnormalised weighted sum of V
    float *out;        // [S][Hq][D]
    uint32_t num_seqs, page_size, num_kv_heads, num_q_heads, head_dim;
    uint32_t unit_tokens, unit_pages, heads_per_group, token_lanes;
    uint32_t cap_units;
    uint32_t group;    // G: query heads per kv head (any positive value)
    uint32_t fused;    // the unit table is rebuilt in LDS (no plan kernel)
    float qscale;      // softmax scale * log2(e)
    Div div_page;
    // Shared-prefix pass (cached loads, matrix-core path): the prefix plan's
    // per-sequence shared pages and runs, and the shared pass's work items.
    uint32_t shared;          // shared work items lead the grid; suffix units follow
    uint32_t pg_area;         // LDS bytes of the staged page IDs (matrix-core kernel)
    // Matrix-core grid with its head groups interleaved: blockIdx.x holds
    // (work index, head group) as x * hg_il + y; 0: the head group is blockIdx.y.
    uint32_t hg_il;
    uint32_t chunk_pages;     // pages of one shared-pass work item
    uint32_t seqs_per_block;  // sequences of one shared work item (four row blocks)
    const uint32_t *pre_pages, *run_of, *work_seq0, *work_chunk, *nwork;
    // int8 pools: one fp32 scale per slot (page * page_size + slot) of each
    const float *k_scales, *v_scales;
};

// 8 stored values (one 16-byte vector) as floats; exact.
template <typename ET>
__device__ __forceinline__ void unpack8(const u32x4 &v, float (&f)[8]) {
    uint32_t w[4];
    __builtin_memcpy(w, &v, sizeof w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (ET::bf16) {
            f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        } else {
            f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
            f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
        }
    }
}

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const unsigned char *p) {
    const u32x4 *v = reinterpret_cast<const u32x4 *>(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(v);
    else
        return *v;
}

template <bool NT>
__device__ __forceinline__ u32x2 ld8(const unsigned char *p) {
    const u32x2 *v = reinterpret_cast<const u32x2 *>(p);
    if constexpr (NT)
        return __builtin_nontemporal_load(v);
    else
        return *v;
}

// Attention over int8 pools with per-slot scales ([Hurray] Per-page-slot
// parameters: every element of a slot's row is its code times the slot's
// scale). A token's scale is common to its whole row, so it comes out of the
// sums: x_t = (scale * sK_t) * sum_d q_d c_td, and V enters as the weight
// p_t * sV_t times the codes. The codes (|c| <= 128) are exact in bf16, so
// the 16-bit products run on the codes themselves; the kernels load 8 codes
// and the slot's scale.
struct Raw8 {
    u32x2 v;  // 8 int8 codes
    float s;  // their slot's scale
};
// 8 int8 codes as the 16-byte vector of their bf16 values (exact).
__device__ __forceinline__ u32x4 codes_bf16(const u32x2 &w) {
    u32x4 o;
    o.x = pack_bf16x2(sbyte(w.x, 0), sbyte(w.x, 1));
    o.y = pack_bf16x2(sbyte(w.x, 2), sbyte(w.x, 3));
    o.z = pack_bf16x2(sbyte(w.y, 0), sbyte(w.y, 1));
    o.w = pack_bf16x2(sbyte(w.y, 2), sbyte(w.y, 3));
    return o;
}
__device__ __forceinline__ u32x4 bits8(const u32x4 &v) { return v; }
__device__ __forceinline__ u32x4 bits8(const Raw8 &r) { return codes_bf16(r.v); }
// 16 codes and their slot's scale: one 16-byte load per lane (the vector
// kernel's int8 layout for head_dim >= 16).
struct Raw16 {
    u32x4 v;
    float s;
};
// Part k (8 elements) of a lane's loaded elements, as 16-bit values.
__device__ __forceinline__ u32x4 part_bits(const u32x4 &v, int) { return v; }
__device__ __forceinline__ u32x4 part_bits(const Raw8 &r, int) { return codes_bf16(r.v); }
__device__ __forceinline__ u32x4 part_bits(const Raw16 &r, int k) {
    return codes_bf16(k ? u32x2{r.v.z, r.v.w} : u32x2{r.v.x, r.v.y});
}
// Word w (4 codes) of a lane's loaded codes.
__device__ __forceinline__ uint32_t code_word(const Raw8 &r, int w) { return w ? r.v.y : r.v.x; }
__device__ __forceinline__ uint32_t code_word(const Raw16 &r, int w) {
    return w == 0 ? r.v.x : w == 1 ? r.v.y : w == 2 ? r.v.z : r.v.w;
}
__device__ __forceinline__ float row_scale(const Raw16 &r) { return r.s; }
// The scale a token's score (or weight) takes: 1 for 16-bit pools.
__device__ __forceinline__ float row_scale(const u32x4 &) { return 1.0f; }
__device__ __forceinline__ float row_scale(const Raw8 &r) { return r.s; }
// Loaded form of 8 elements: the 16-bit values themselves, or codes + scale.
template <bool Q8>
using Loaded8 = std::conditional_t<Q8, Raw8, u32x4>;
// Loaded form of a vector-kernel lane's EPL elements.
template <bool Q8, int EPL>
using LoadedE = std::conditional_t<!Q8, u32x4, std::conditional_t<EPL == 16, Raw16, Raw8>>;
// Bytes per stored element.
template <bool Q8>
constexpr uint32_t elem_bytes() { return Q8 ? 1 : 2; }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// x from another lane of the same 16-lane row, by a DPP pattern (a plain
// VALU operand, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over the LPH lanes of a lane group (aligned groups of LPH lanes); every
// lane of the group gets the same value, since each step adds a lane's value
// to its partner's and IEEE addition is commutative.
template <int LPH, bool SHFL>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (SHFL) {
        // through the LDS crossbar, beside the VALU: measured faster with one
        // query head per kv head, where few independent sums can hide the DPP
        // hazards
#pragma unroll
        for (int o = LPH / 2; o >= 1; o >>= 1)
            x += __shfl_xor(x, o, 64);
        return x;
    }
    if constexpr (LPH >= 2)
        x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPH >= 4)
        x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPH >= 8)
        x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8 lanes
    if constexpr (LPH >= 16)
        x += dpp<0x140>(x);  // row_mirror: the other 8 lanes of the 16-lane row
    if constexpr (LPH >= 32)
        x += __shfl_xor(x, 16, 64);
    return x;
}

// Sum over the 8 stored elements of q (packed) times k (packed), fp32
// accumulation: v_dot2 takes two 16-bit products per instruction.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short bf16x2_bits __attribute__((ext_vector_type(2)));
template <typename ET>
__device__ __forceinline__ float dot8(const uint32_t (&q)[4], const u32x4 &k, float d = 0.0f) {
    uint32_t w[4];
    __builtin_memcpy(w, &k, sizeof w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (ET::bf16)
            d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_bits, q[i]),
                                                __builtin_bit_cast(bf16x2_bits, w[i]), d, false);
        else
            d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, q[i]),
                                       __builtin_bit_cast(f16x2, w[i]), d, false);
    }
    return d;
}

// Tokens per batch of one lane group: all their K and V loads are in flight
// together. Fewer for larger groups, whose query and accumulator registers
// grow with G.
#ifndef HP_ATTN_BATCH_LARGE_GROUP
#define HP_ATTN_BATCH_LARGE_GROUP 4
#endif
template <int GT>
constexpr int batch_tokens() {
    return GT <= 2 ? 8 : (GT == 4 ? 4 : HP_ATTN_BATCH_LARGE_GROUP);
}

// Units of sequence s: ceil(L_s / U).
template <typename IdxT>
__device__ __forceinline__ uint32_t units_of_seq(const void *seq_lens, uint32_t s, uint32_t U) {
    const uint64_t len = ld_idx<IdxT>(seq_lens, s);
    return (uint32_t)(len / U + (len % U != 0));
}

// unit_end[s] for all S sequences into LDS (inclusive running unit count,
// capped at cap), by the whole workgroup: each thread sums a contiguous run
// of sequences, a shuffle scan per wave and the wave totals through LDS give
// each run's start. Ends with a barrier.
template <typename IdxT>
__device__ __forceinline__ void unit_scan_lds(const void *seq_lens, uint32_t S, uint32_t U,
                                              uint32_t cap, uint32_t *ue) {
    __shared__ uint32_t wave_sum[kAttnThreads / 64];
    const uint32_t per = (S + kAttnThreads - 1) / kAttnThreads;
    const uint32_t i0 = min32(S, threadIdx.x * per), i1 = min32(S, i0 + per);
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t v = 0;
    for (uint32_t i = i0; i < i1; ++i)
        v += units_of_seq<IdxT>(seq_lens, i, U);
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= (uint32_t)o)
            incl += y;
    }
    if (lane == 63)
        wave_sum[wave] = incl;
    __syncthreads();
    uint32_t run = incl - v;
    for (uint32_t w = 0; w < wave; ++w)
        run += wave_sum[w];
    for (uint32_t i = i0; i < i1; ++i) {
        run += units_of_seq<IdxT>(seq_lens, i, U);
        ue[i] = min32(run, cap);
    }
    __syncthreads();
}

// GT query-head slots per lane group (1, 2, 4 or 8 >= G, or 8 with grid z
// chunks of 8 query heads when G > 8); slots past G are computed and dropped.
// Q8: int8 pools with per-slot scales (ET is then BF16). EPL: elements per
// lane, 8 (one 16-byte vector of 16-bit values, or 8 codes), or 16 codes
// (one 16-byte load) for int8 pools with head_dim >= 16.
template <typename ET, typename IdxT, int LPH, int GT, bool NT, bool Q8, int EPL>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(AArgs a) {
    // No implicit multiply-add fusion: each fused step below is an explicit
    // fma, and a score must round before its max is subtracted, so that the
    // largest score weighs exactly exp2(0) = 1.
#pragma clang fp contract(off)
    constexpr int TB = batch_tokens<GT>();
    constexpr uint32_t NG = kAttnThreads / LPH;  // lane groups
    constexpr uint32_t D = LPH * EPL;
    constexpr int NP = EPL / 8;  // 8-element parts per lane
    static_assert(EPL == 8 || (Q8 && EPL == 16), "16 elements per lane only for int8 pools");
    extern __shared__ __align__(16) unsigned char lds[];
    const uint32_t S = a.num_seqs;
    // LDS: [unit_end (fused)] [page IDs of the unit] [token-lane merge]
    const size_t ue_bytes = a.fused ? ((4 * (size_t)S + 15) & ~(size_t)15) : 0;
    uint32_t *ue_lds = reinterpret_cast<uint32_t *>(lds);
    uint64_t *pages = reinterpret_cast<uint64_t *>(lds + ue_bytes);
    float *red = reinterpret_cast<float *>(lds + ue_bytes + 8 * (size_t)a.unit_pages);
    const uint32_t *unit_end = a.unit_end;
    if (a.fused) {
        unit_scan_lds<IdxT>(a.seq_lens, S, a.unit_tokens, a.cap_units, ue_lds);
        unit_end = ue_lds;
    }

    const uint32_t g = blockIdx.x;
    const uint32_t total = uni(unit_end[S - 1]);
    const uint32_t Hq = a.num_q_heads, Hkv = a.num_kv_heads, P = a.page_size;
    const uint32_t hpw = a.heads_per_group, G = a.group;
    const uint32_t hq0 = blockIdx.y * hpw * G;  // this group's first query head
    const uint32_t nq = (min32(Hkv, (blockIdx.y + 1) * hpw) - blockIdx.y * hpw) * G;
    const uint32_t gz = blockIdx.z * GT;          // first slot's offset in the kv head's group
    if (g >= total) {
        // spare workgroups: workgroup total + s writes the zeros of sequence s
        // when it has no token (no unit would write them)
        const uint32_t se = g - total;
        if (se >= S || blockIdx.z != 0 || ld_idx<IdxT>(a.seq_lens, se) != 0)
            return;
        float *o = a.out + ((uint64_t)se * Hq + hq0) * D;
        for (uint32_t e = threadIdx.x; e < nq * D; e += kAttnThreads)
            o[e] = 0.0f;
        return;
    }
    uint32_t s;
    if (a.fused) {
        uint32_t lo = 0, hi = S - 1;  // first sequence whose units reach past g
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (ue_lds[mid] > g)
                hi = mid;
            else
                lo = mid + 1;
        }
        s = uni(lo);
    } else {
        s = uni(a.unit_seq[g]);
    }
    const uint32_t u0 = s ? uni(unit_end[s - 1]) : 0;
    const uint64_t L = uni64(ld_idx<IdxT>(a.seq_lens, s));
    const uint64_t sp0 = uni64(ld_idx<IdxT>(a.seq_ptr, s));
    const uint64_t t0 = (uint64_t)(g - u0) * a.unit_tokens;  // a multiple of the page size
    if (t0 >= L)
        return;  // only when total_tokens disagrees with the counts: read nothing
    const uint32_t n = (uint32_t)min64(L - t0, a.unit_tokens);
    const uint64_t pg0 = t0 / a.page_size;
    const uint32_t npg = udiv32(n + a.page_size - 1, a.div_page);
    for (uint32_t i = threadIdx.x; i < npg; i += kAttnThreads)
        pages[i] = ld_idx<IdxT>(a.block_table, sp0 + pg0 + i);
    __syncthreads();

    const uint32_t lane = threadIdx.x;
    const uint32_t lg = lane / LPH, r = lane % LPH;
    const uint32_t TL = a.token_lanes;
    const uint32_t hl = lg % hpw, tl = lg / hpw;
    const uint32_t h = blockIdx.y * hpw + hl;
    const bool active = tl < TL && h < Hkv;

    float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
    for (int gi = 0; gi < GT; ++gi) {
        m[gi] = -__builtin_inff();
        l[gi] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[gi][e] = 0.0f;
    }

    if (active) {
        uint32_t qp[GT][NP][4];  // the query's EPL elements of this lane, packed as stored
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            const uint32_t c = min32(gz + gi, G - 1);  // slots past G repeat the last head
            const uint64_t qo = (((uint64_t)s * Hq + (uint64_t)h * G + c) * D + r * EPL) * 2;
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                const u32x4 v = ld16<false>(a.q + qo + 16 * k);
                __builtin_memcpy(qp[gi][k], &v, 16);
            }
        }
        const uint64_t head_off = ((uint64_t)h * D + r * EPL) * elem_bytes<Q8>();
        const uint64_t slot_bytes = (uint64_t)Hkv * D * elem_bytes<Q8>();
        // each batch starts with a token in range, so its running max is finite
        for (uint32_t jb = 0; jb + tl < n; jb += TB * TL) {
            LoadedE<Q8, EPL> kq[TB], vq[TB];
            bool ok[TB];
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                const uint32_t j = jb + tl + i * TL;
                ok[i] = j < n;
                const uint32_t jj = ok[i] ? j : n - 1;  // always a real row: loads need no guard
                const uint32_t pj = udiv32(jj, a.div_page);
                const uint64_t row = pages[pj] * P + (jj - pj * P);
                const uint64_t off = row * slot_bytes + head_off;
                if constexpr (Q8 && EPL == 16) {
                    kq[i] = Raw16{ld16<NT>(a.k_pool + off), a.k_scales[row]};
                    vq[i] = Raw16{ld16<NT>(a.v_pool + off), a.v_scales[row]};
                } else if constexpr (Q8) {
                    kq[i] = Raw8{ld8<NT>(a.k_pool + off), a.k_scales[row]};
                    vq[i] = Raw8{ld8<NT>(a.v_pool + off), a.v_scales[row]};
                } else {
                    kq[i] = ld16<NT>(a.k_pool + off);
                    vq[i] = ld16<NT>(a.v_pool + off);
                }
            }
            float x[GT][TB];
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                u32x4 kb[NP];
#pragma unroll
                for (int k = 0; k < NP; ++k)
                    kb[k] = part_bits(kq[i], k);
                // int8 pools: the token's K scale joins the softmax scale
                const float xs = Q8 ? a.qscale * row_scale(kq[i]) : a.qscale;
#pragma unroll
                for (int gi = 0; gi < GT; ++gi) {
                    float d = dot8<ET>(qp[gi][0], kb[0]);
#pragma unroll
                    for (int k = 1; k < NP; ++k)
                        d = dot8<ET>(qp[gi][k], kb[k], d);
                    const float dot = group_sum<LPH, GT == 1>(d) * xs;
                    x[gi][i] = ok[i] ? dot : -__builtin_inff();
                }
            }
            float p[GT][TB];
#pragma unroll
            for (int gi = 0; gi < GT; ++gi) {
                float mx = m[gi];
#pragma unroll
                for (int i = 0; i < TB; ++i)
                    mx = __builtin_fmaxf(mx, x[gi][i]);
                // mx is finite (the batch's first token is in range); m may be -inf
                const float corr = exp2_hw(m[gi] - mx);
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < TB; ++i) {
                    p[gi][i] = ok[i] ? exp2_hw(x[gi][i] - mx) : 0.0f;
                    ps += p[gi][i];
                }
                l[gi] = l[gi] * corr + ps;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[gi][e] *= corr;
                m[gi] = mx;
            }
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                float vf[EPL];
                if constexpr (Q8) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e)  // the codes (exact)
                        vf[e] = sbyte(code_word(vq[i], e / 4), e & 3);
                } else {
                    unpack8<ET>(vq[i], vf);
                }
#pragma unroll
                for (int gi = 0; gi < GT; ++gi) {
                    // int8 pools: the weight times the token's V scale (the sum
                    // of weights l stays unscaled)
                    const float pv = Q8 ? p[gi][i] * row_scale(vq[i]) : p[gi][i];
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[gi][e] = __builtin_fmaf(pv, vf[e], acc[gi][e]);
                }
            }
        }
    }

    // Merge the token lanes of each head into token lane 0.
    if (TL > 1) {
        float *rml = red;                  // [NG][2]
        float *racc = red + 2 * NG;        // [NG][D]
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            if (gz + gi >= G)
                break;  // uniform: slots past G are not merged
            if (active && tl > 0) {
                if (r == 0) {
                    rml[2 * lg] = m[gi];
                    rml[2 * lg + 1] = l[gi];
                }
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    racc[lg * D + r * EPL + e] = acc[gi][e];
            }
            __syncthreads();
            if (active && tl == 0) {
                float M = m[gi];
                for (uint32_t t2 = 1; t2 < TL; ++t2)
                    M = __builtin_fmaxf(M, rml[2 * (t2 * hpw + hl)]);
                const float c0 = exp2_hw(m[gi] - M);
                l[gi] *= c0;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[gi][e] *= c0;
                for (uint32_t t2 = 1; t2 < TL; ++t2) {
                    const uint32_t o = t2 * hpw + hl;
                    const float mo = rml[2 * o];
                    // a token lane that saw no token has max -inf and weight 0
                    const float c = mo == -__builtin_inff() ? 0.0f : exp2_hw(mo - M);
                    l[gi] = __builtin_fmaf(rml[2 * o + 1], c, l[gi]);
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[gi][e] = __builtin_fmaf(racc[o * D + r * EPL + e], c, acc[gi][e]);
                }
                m[gi] = M;
            }
            __syncthreads();
        }
    }

    const uint32_t units = uni(unit_end[s]) - u0;
    if (units == 1) {
        // the sequence's only unit: normalise and write the output directly
        if (active && tl == 0) {
#pragma unroll
            for (int gi = 0; gi < GT; ++gi) {
                if (gz + gi >= G)
                    break;
                float *dst = a.out + ((uint64_t)s * Hq + (uint64_t)h * G + gz + gi) * D + r * EPL;
                float o[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    o[e] = acc[gi][e] / l[gi];
#pragma unroll
                for (int k = 0; k < EPL / 4; ++k) {
                    u32x4 v;
                    __builtin_memcpy(&v, &o[4 * k], 16);
                    reinterpret_cast<u32x4 *>(dst)[k] = v;
                }
            }
        }
        return;
    }

    if (active && tl == 0) {
#pragma unroll
        for (int gi = 0; gi < GT; ++gi) {
            if (gz + gi >= G)
                break;
            const uint64_t idx = (uint64_t)g * Hq + (uint64_t)h * G + gz + gi;
            float *dst = a.part_acc + idx * D + r * EPL;
#pragma unroll
            for (int k = 0; k < EPL / 4; ++k) {
                u32x4 v;
                __builtin_memcpy(&v, &acc[gi][4 * k], 16);
                reinterpret_cast<u32x4 *>(dst)[k] = v;
            }
            if (r == 0) {
                a.part_ml[2 * idx] = m[gi];
                a.part_ml[2 * idx + 1] = l[gi];
            }
        }
    }
}

// ---- grouped query heads on the matrix cores -----------------------------------
//
// With G >= 2 query heads per kv head, a unit's scores are a (G x D) by
// (D x tokens) product and its output a (G x tokens) by (tokens x D) one, so
// they run on v_mfma_f32_16x16x32 (bf16 or f16 inputs, fp32 accumulation),
// the G query heads as the 16 rows of the matrix (rows past G are zero and
// dropped). One wave per kv head; a workgroup takes 4 kv heads of one unit.
// Per tile of 32 tokens:
//  * scores, two 16-token blocks: K is loaded as whole head rows, staged in
//    the wave's LDS tile buffer, and read from there into the B layout (16
//    contiguous bytes of one token's row per lane);
//  * per-row online softmax in base 2 on the accumulator layout (a lane holds
//    4 rows of one token), row maxima and sums by DPP within 16-lane rows;
//  * weights times V: the weights go through LDS into the A layout and are
//    split into three bf16 (or f16) parts whose sum is the binary32 weight, so
//    the product keeps binary32 weights; V goes through LDS as 288-byte token
//    rows and reaches the B layout by 16-bit reads. Inside the tile, lane
//    group g takes tokens g, g + 4, ..., g + 28 on both sides (the sum over
//    tokens is the same in any order), which spreads the four groups' reads
//    over disjoint LDS banks.
// Partial results and outputs have the vector kernel's format (max and sum in
// base 2, unnormalised sums of V), so the combine kernel serves both.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMfmaTile = 32;   // tokens per tile (the contraction of weights x V)
constexpr uint32_t kMfmaRows = 16;   // query-head rows of one MFMA
constexpr uint32_t kMfmaWaves = kAttnThreads / 64;  // kv heads per workgroup
constexpr uint32_t kPRow = 36;       // floats per weight row in LDS (bank skew)

template <typename ET> struct Mma;
template <> struct Mma<BF16> {
    using V8 = bf16x8;
    using E = __bf16;
    static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ __bf16 narrow(float x) { return (__bf16)x; }
};
template <> struct Mma<F16> {
    using V8 = f16x8;
    using E = _Float16;
    static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ _Float16 narrow(float x) { return (_Float16)x; }
};

// Bytes per token row of a wave's V tile in LDS: the row plus 32 (rows four
// tokens apart then start 8 banks apart).
template <int D>
constexpr uint32_t v_row_bytes() { return D * 2 + 32; }
// LDS of one wave: its V tile and its weight tile.
template <int D>
constexpr size_t mfma_wave_lds() { return kMfmaTile * v_row_bytes<D>() + kMfmaRows * kPRow * 4; }

// Maximum and sum over the 16 lanes of a DPP row (the lanes that hold one
// accumulator row's 16 tokens); every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float x) {
    x = __builtin_fmaxf(x, dpp<0xB1>(x));
    x = __builtin_fmaxf(x, dpp<0x4E>(x));
    x = __builtin_fmaxf(x, dpp<0x141>(x));
    return __builtin_fmaxf(x, dpp<0x140>(x));
}

// Orders this wave's LDS writes before its other lanes' reads (a wave's LDS
// operations complete in order once waited for; the clobber keeps the
// compiler from moving memory accesses across).
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Query head of matrix row r (and the row of query head q): r = 4 (q % 4) +
// q / 4, an involution on 0..15. A lane holds the accumulator rows 4 grp + i,
// that is query heads 4 i + grp, so with G <= 4 (G <= 8) every live row sits
// at i = 0 (i < 2) and the softmax of the others is skipped.
__device__ __forceinline__ uint32_t row_head(uint32_t r) { return 4 * (r & 3) + (r >> 2); }

// The unit's n tokens of kv head h against the query rows in qa: the online
// softmax state m, l and the unnormalised output o of the rows this lane
// holds (rows 4 grp + i for i < R, columns 16 db + c16). page_off: the byte
// offsets in the pools of the unit's pages, staged in LDS (with Q8, int8
// pools: the index of each page's first slot, page * page_size, which also
// indexes the scales). vt, pt: this wave's V and weight tiles in LDS.
template <typename ET, int D, bool NT, int R, bool Q8>
__device__ __forceinline__ void mfma_span(const AArgs &a, const uint64_t *page_off, uint32_t n,
                                          uint32_t h,
                                          const typename Mma<ET>::V8 (&qa)[D / 32],
                                          unsigned char *vt, float *pt, float (&m)[4],
                                          float (&l)[4], f32x4 (&o)[D / 16]) {
#pragma clang fp contract(off)
    using M = Mma<ET>;
    using V8 = typename M::V8;
    constexpr uint32_t KK = D / 32;  // MFMAs per 16-token score block
    constexpr uint32_t DB = D / 16;  // 16-column blocks of the output
    constexpr uint32_t VRB = v_row_bytes<D>();
    const uint32_t lane = threadIdx.x & 63, P = a.page_size, Hkv = a.num_kv_heads;
    const uint32_t c16 = lane & 15, grp = lane >> 4;
    const uint32_t slot_bytes = Hkv * D * elem_bytes<Q8>();
    const uint32_t head_off = h * D * elem_bytes<Q8>();

    // Loads take whole head rows: chunk c of a tile is 16 bytes for each of
    // the 64 lanes, lane L reading bytes 16 (L % (D / 8)) of the head row of
    // token 4 c + L / (D / 8) (D = 128; the same form at D = 64), so a load
    // covers a few complete 256-byte rows rather than 64-byte pieces of 16
    // rows (half as many cache-line requests per byte; measured on MI355X,
    // decode batch with four query heads per kv head: 244 us with the pieces,
    // 198 us with whole rows for both K and V). K and V both go through the wave's
    // tile buffer in LDS, K on to the B layout of the score product. Tokens
    // past n repeat the last token (a real row; masked below).
    // (int8 pools: chunk c is 16 codes for each lane, lane L reading codes
    // 16 (L % (D / 16)) of the head row of token 8 c + L / (D / 16) (D = 128),
    // which become 32 bytes of bf16 on the way into LDS; and lane i < 32
    // loads the scale of the tile's token i, which the score and the weight
    // of that token take)
    V8 kb[2][KK];
    constexpr uint32_t C16 = Q8 ? 1 : 2 * KK, C8 = Q8 ? KK : 1;
    u32x4 kc[C16], vc[C16];
    u32x4 kc8[C8], vc8[C8];
    float ksc = 0.0f, vsc = 0.0f;
    auto load_rows = [&](const unsigned char *pool, const float *scales, uint32_t tb,
                         u32x4 (&d16)[C16], u32x4 (&d8)[C8], float &dsc) {
        if constexpr (Q8) {
#pragma unroll
            for (uint32_t c = 0; c < KK; ++c) {
                const uint32_t ch = 64 * c + lane;
                const uint32_t jt = ch / (D / 16), dc = ch % (D / 16);
                const uint32_t j = min32(tb + jt, n - 1);
                const uint32_t pj = udiv32(j, a.div_page);
                d8[c] = ld16<NT>(pool + (page_off[pj] + (j - pj * P)) * slot_bytes + head_off +
                                 16 * dc);
            }
            const uint32_t j = min32(tb + (lane & (kMfmaTile - 1)), n - 1);
            const uint32_t pj = udiv32(j, a.div_page);
            dsc = scales[page_off[pj] + (j - pj * P)];
        } else {
#pragma unroll
            for (uint32_t c = 0; c < 2 * KK; ++c) {
                const uint32_t ch = 64 * c + lane;
                const uint32_t jt = ch / (D / 8), dc = ch % (D / 8);
                const uint32_t j = min32(tb + jt, n - 1);
                const uint32_t pj = udiv32(j, a.div_page);
                d16[c] = ld16<NT>(pool + page_off[pj] + (uint64_t)(j - pj * P) * slot_bytes +
                                  head_off + 16 * dc);
            }
        }
    };
    // token-major rows of VRB bytes
    auto store_rows = [&](const u32x4 (&s16)[C16], const u32x4 (&s8)[C8]) {
        if constexpr (Q8) {
#pragma unroll
            for (uint32_t c = 0; c < KK; ++c) {
                const uint32_t ch = 64 * c + lane;
                const uint32_t jt = ch / (D / 16), dc = ch % (D / 16);
                u32x4 *dst = reinterpret_cast<u32x4 *>(vt + jt * VRB + 32 * dc);
                dst[0] = codes_bf16(u32x2{s8[c].x, s8[c].y});
                dst[1] = codes_bf16(u32x2{s8[c].z, s8[c].w});
            }
        } else {
#pragma unroll
            for (uint32_t c = 0; c < 2 * KK; ++c) {
                const uint32_t ch = 64 * c + lane;
                const uint32_t jt = ch / (D / 8), dc = ch % (D / 8);
                *reinterpret_cast<u32x4 *>(vt + jt * VRB + 16 * dc) = s16[c];
            }
        }
    };
    // K of the tile into the B layout: the lane's token 16 b + c16, bytes
    // 64 kk + 16 grp of its row
    auto stage_k = [&]() {
        wave_lds_sync();  // the previous tile's reads of the buffer are done
        store_rows(kc, kc8);
        wave_lds_sync();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (uint32_t kk = 0; kk < KK; ++kk)
                kb[b][kk] = *reinterpret_cast<const V8 *>(vt + (16 * b + c16) * VRB + 64 * kk +
                                                           16 * grp);
    };
    // Software pipeline: tile tb + 32's K loads follow tile tb's score
    // products (which free the K registers), and its V loads follow tile tb's
    // V writes to LDS, so they are in flight during the softmax and the
    // weights x V products. The last tile is a separate copy (no prefetch)
    // so that the loop body has no branch around its loads.
    auto tile = [&](uint32_t tb, auto more_tag) {
        constexpr bool more = decltype(more_tag)::value;
        stage_k();
        // scores: lane holds rows 4 grp + i of token tb + 16 b + c16
        float x[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (uint32_t kk = 0; kk < KK; ++kk)
                acc = M::mma(qa[kk], kb[b][kk], acc);
            const bool ok = tb + 16 * b + c16 < n;
            // int8 pools: the K scale of token 16 b + c16 joins the softmax scale
            const float xs = Q8 ? a.qscale * __shfl(ksc, (int)(16 * b + c16), 64) : a.qscale;
#pragma unroll
            for (int i = 0; i < R; ++i)
                x[b][i] = ok ? acc[i] * xs : -__builtin_inff();
        }
        if constexpr (more)
            load_rows(a.k_pool, a.k_scales, tb + kMfmaTile, kc, kc8, ksc);
        // online softmax per row (the tile's first token is in range, so the
        // new maximum is finite). When no row's maximum grows the correction
        // is exactly 1 and the rescaling is skipped (bit-identical).
        float p[2][4], mx[4];
        bool grow = false;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            mx[i] = __builtin_fmaxf(m[i], row16_max(__builtin_fmaxf(x[0][i], x[1][i])));
            grow |= mx[i] != m[i];
            p[0][i] = exp2_hw(x[0][i] - mx[i]);
            p[1][i] = exp2_hw(x[1][i] - mx[i]);
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float corr = exp2_hw(m[i] - mx[i]);
                l[i] = l[i] * corr;
#pragma unroll
                for (uint32_t db = 0; db < DB; ++db)
                    o[db][i] *= corr;
                m[i] = mx[i];
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
            l[i] = l[i] + group_sum<16, false>(p[0][i] + p[1][i]);
        // the previous tile's LDS reads are done before this tile's writes
        wave_lds_sync();
        // weights to LDS in the A layout: token t of the tile goes to column
        // 8 (t % 4) + t / 4 (rows i >= R are not written: their output rows
        // are never read)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t t = 16 * b + c16;
            const uint32_t col = 8 * (t & 3) + (t >> 2);
            // int8 pools: the weight times the token's V scale (l stays unscaled)
            const float vs = Q8 ? __shfl(vsc, (int)t, 64) : 1.0f;
#pragma unroll
            for (int i = 0; i < R; ++i)
                pt[(4 * grp + i) * kPRow + col] = Q8 ? p[b][i] * vs : p[b][i];
        }
        // V tile to LDS (the buffer's K reads are done: the score products
        // consumed them)
        store_rows(vc, vc8);
        wave_lds_sync();
        if constexpr (more)
            load_rows(a.v_pool, a.v_scales, tb + kMfmaTile, vc, vc8, vsc);
        // weights as three A operands whose sum is the binary32 weight
        V8 pa[3];
        {
            float w[8];
            __builtin_memcpy(&w[0], pt + c16 * kPRow + 8 * grp, 16);
            __builtin_memcpy(&w[4], pt + c16 * kPRow + 8 * grp + 4, 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const auto hi = M::narrow(w[e]);
                const float r1 = w[e] - (float)hi;
                const auto mid = M::narrow(r1);
                const float r2 = r1 - (float)mid;
                pa[0][e] = hi;
                pa[1][e] = mid;
                pa[2][e] = M::narrow(r2);
            }
        }
        // output += weights x V, 16 columns at a time; lane group grp reads
        // tokens grp + 4 e of column 16 db + c16
#pragma unroll
        for (uint32_t db = 0; db < DB; ++db) {
            V8 vb;
            const unsigned char *vr = vt + (16 * db + c16) * 2 + grp * VRB;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vb[e] = *reinterpret_cast<const typename M::E *>(vr + 4 * e * VRB);
#pragma unroll
            for (int k = 0; k < 3; ++k)
                o[db] = M::mma(pa[k], vb, o[db]);
        }
    };
    load_rows(a.k_pool, a.k_scales, 0, kc, kc8, ksc);
    load_rows(a.v_pool, a.v_scales, 0, vc, vc8, vsc);
    uint32_t tb = 0;
    for (; tb + kMfmaTile < n; tb += kMfmaTile)
        tile(tb, std::integral_constant<bool, true>());
    tile(tb, std::integral_constant<bool, false>());  // n >= 1: the unit's last tile
}

// ---- shared-prefix pass ---------------------------------------------------------
//
// [Hurray] Prefix Sharing: slices may name the same leading pages, and then
// every sequence that shares them attends over the same K and V rows.
// Sequences are taken in runs: consecutive sequences whose slices begin with
// at least kMinSharedTokens tokens of identical full pages (both sequences'
// counts cover them); a run's shared part is the shortest such common prefix
// in it, which every member holds. The shared part is computed once per kv
// head, chunk of kSharedChunkTokens tokens and item of seqs_per_block
// sequences of the run: the workgroup's four waves take four row blocks (the
// query heads of 16 / G sequences each, stacked as the matrix core's 16 rows;
// one sequence and 16 of its query heads per block when G > 16), and all 256
// threads load each K/V tile once, as whole head rows, into a double-buffered
// LDS tile that the four waves read. A sequence's units are its shared chunks followed by units
// over the tokens after the shared part; the shared pass writes the partial
// results of the first kind into those units' slots, the attention kernel the
// rest, and the combine kernel merges them as before.

// Tokens of one shared work item (about: whole pages). Measured on MI355X,
// prefix batch (1,024 shared tokens), G = 4 / 8: 256 -> 112.8 / 146.7 us,
// 512 -> 99.9 / 124.1 us (fewer partial results to merge), 1,024 -> 113.0 /
// 132.1 us (too few work items to overlap the units).
#ifndef HP_ATTN_SHARED_CHUNK_TOKENS
#define HP_ATTN_SHARED_CHUNK_TOKENS 512
#endif
constexpr uint32_t kSharedChunkTokens = HP_ATTN_SHARED_CHUNK_TOKENS;
constexpr uint32_t kMinSharedTokens = 64;     // two matrix tiles

// One 32-token tile of a wave against K and V tiles in LDS (token-major
// rows of v_row_bytes): the online softmax of all 16 rows, as in mfma_span.
// Q8: the tiles hold int8 codes as bf16, and kss / vss the tile's 32 K and V
// scales.
template <typename ET, int D, bool Q8>
__device__ __forceinline__ void lds_tile(const AArgs &a, const unsigned char *kt,
                                         const unsigned char *vt, const float *kss,
                                         const float *vss, float *pt, uint32_t tb, uint32_t n,
                                         const typename Mma<ET>::V8 (&qa)[D / 32],
                                         float (&m)[4], float (&l)[4], f32x4 (&o)[D / 16]) {
#pragma clang fp contract(off)
    using M = Mma<ET>;
    using V8 = typename M::V8;
    constexpr uint32_t KK = D / 32;
    constexpr uint32_t DB = D / 16;
    constexpr uint32_t VRB = v_row_bytes<D>();
    const uint32_t lane = threadIdx.x & 63, c16 = lane & 15, grp = lane >> 4;
    float x[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (uint32_t kk = 0; kk < KK; ++kk)
            acc = M::mma(qa[kk],
                         *reinterpret_cast<const V8 *>(kt + (16 * b + c16) * VRB + 64 * kk +
                                                       16 * grp),
                         acc);
        const bool ok = tb + 16 * b + c16 < n;
        const float xs = Q8 ? a.qscale * kss[16 * b + c16] : a.qscale;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[b][i] = ok ? acc[i] * xs : -__builtin_inff();
    }
    float p[2][4], mx[4];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mx[i] = __builtin_fmaxf(m[i], row16_max(__builtin_fmaxf(x[0][i], x[1][i])));
        grow |= mx[i] != m[i];
        p[0][i] = exp2_hw(x[0][i] - mx[i]);
        p[1][i] = exp2_hw(x[1][i] - mx[i]);
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float corr = exp2_hw(m[i] - mx[i]);
            l[i] = l[i] * corr;
#pragma unroll
            for (uint32_t db = 0; db < DB; ++db)
                o[db][i] *= corr;
            m[i] = mx[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        l[i] = l[i] + group_sum<16, false>(p[0][i] + p[1][i]);
    wave_lds_sync();  // the previous tile's reads of pt are done
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const uint32_t t = 16 * b + c16;
        const uint32_t col = 8 * (t & 3) + (t >> 2);
        const float vs = Q8 ? vss[t] : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pt[(4 * grp + i) * kPRow + col] = Q8 ? p[b][i] * vs : p[b][i];
    }
    wave_lds_sync();
    V8 pa[3];
    {
        float w[8];
        __builtin_memcpy(&w[0], pt + c16 * kPRow + 8 * grp, 16);
        __builtin_memcpy(&w[4], pt + c16 * kPRow + 8 * grp + 4, 16);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const auto hi = M::narrow(w[e]);
            const float r1 = w[e] - (float)hi;
            const auto mid = M::narrow(r1);
            const float r2 = r1 - (float)mid;
            pa[0][e] = hi;
            pa[1][e] = mid;
            pa[2][e] = M::narrow(r2);
        }
    }
#pragma unroll
    for (uint32_t db = 0; db < DB; ++db) {
        V8 vb;
        const unsigned char *vr = vt + (16 * db + c16) * 2 + grp * VRB;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vb[e] = *reinterpret_cast<const typename M::E *>(vr + 4 * e * VRB);
#pragma unroll
        for (int k = 0; k < 3; ++k)
            o[db] = M::mma(pa[k], vb, o[db]);
    }
}

// Work item w, kv head h: chunk work_chunk[w] of the item of seqs_per_block
// sequences that begins at sequence work_seq0[w] (and query-head chunk z
// when G > 16). Called by whole workgroups.
template <typename ET, typename IdxT, int D, bool Q8>
__device__ __forceinline__ void shared_item(const AArgs &a, uint32_t w, uint32_t h,
                                            unsigned char *lds) {
#pragma clang fp contract(off)
    using M = Mma<ET>;
    using V8 = typename M::V8;
    constexpr uint32_t KK = D / 32;
    constexpr uint32_t DB = D / 16;
    constexpr uint32_t VRB = v_row_bytes<D>();
    constexpr uint32_t CPT = kMfmaTile * D / 8 / kAttnThreads;  // 16-byte chunks per thread
    const uint32_t s0 = uni(a.work_seq0[w]), c = uni(a.work_chunk[w]);
    const uint32_t run = uni(a.run_of[s0]), C = uni(a.pre_pages[s0]);
    const uint32_t S = a.num_seqs, Hq = a.num_q_heads, Hkv = a.num_kv_heads, P = a.page_size;
    const uint32_t G = a.group, spb = a.seqs_per_block / kMfmaWaves;  // sequences per wave
    const uint32_t pg0 = c * a.chunk_pages;
    const uint32_t npg = min32(C - pg0, a.chunk_pages);  // whole pages, all tokens live
    const uint32_t n = npg * P;
    const uint32_t slot_bytes = Hkv * D * elem_bytes<Q8>(), head_off = h * D * elem_bytes<Q8>();
    // byte offsets of the pages (int8 pools: their first slots)
    uint64_t *pages = reinterpret_cast<uint64_t *>(lds);
    const uint64_t sp0 = uni64(ld_idx<IdxT>(a.seq_ptr, s0));
    const uint64_t page_mul = Q8 ? (uint64_t)P : (uint64_t)P * slot_bytes;
    for (uint32_t i = threadIdx.x; i < npg; i += kAttnThreads)
        pages[i] = ld_idx<IdxT>(a.block_table, sp0 + pg0 + i) * page_mul;
    __syncthreads();

    // LDS: K and V tiles of two stages in the four wave regions (stage b: K
    // in region 2 b, V in region 2 b + 1), each wave's weight tile after its
    // region's tile
    unsigned char *region = lds + a.pg_area;
    constexpr uint32_t WL = (uint32_t)mfma_wave_lds<D>();
    // int8 pools: the K and V scales of each stage's 32 tokens, after the tiles
    float *scl = reinterpret_cast<float *>(region + kMfmaWaves * WL);  // [stage][K, V][32]
    const uint32_t wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    float *pt = reinterpret_cast<float *>(region + wave * WL + kMfmaTile * VRB);
    const uint32_t c16 = lane & 15, grp = lane >> 4;
    // Row r of this wave: with G <= 16, query head r % G of sequence
    // s0 + spb wave + r / G; with G > 16, query head 16 z + r of sequence
    // s0 + wave. A row is live when its sequence belongs to the run.
    auto row_seq = [&](uint32_t r, uint32_t &seq, uint32_t &qi) -> bool {
        if (G <= kMfmaRows) {
            const uint32_t k = r / G;
            seq = s0 + spb * wave + k;
            qi = r - k * G;
            return k < spb && seq < S && a.run_of[seq] == run;
        }
        seq = s0 + wave;
        qi = blockIdx.z * kMfmaRows + r;
        return qi < G && seq < S && a.run_of[seq] == run;
    };
    V8 qa[KK];
    {
        uint32_t seq, qi;
        const bool live = row_seq(c16, seq, qi);
        const uint64_t qo = live ? (((uint64_t)seq * Hq + (uint64_t)h * G + qi) * D + 8 * grp) * 2
                                 : 0;
#pragma unroll
        for (uint32_t kk = 0; kk < KK; ++kk) {
            u32x4 v = ld16<false>(a.q + qo + kk * 64);
            if (!live)
                v = u32x4(0);
            qa[kk] = __builtin_bit_cast(V8, v);
        }
    }
    float m[4], l[4];
    f32x4 o[DB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m[i] = -__builtin_inff();
        l[i] = 0.0f;
    }
#pragma unroll
    for (uint32_t db = 0; db < DB; ++db)
        o[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // thread t loads chunk t + 256 e of the tile: 16 bytes of the head row of
    // token (t + 256 e) / (D / 8), so a wave's load covers whole rows
    // (int8 pools: 8 bytes of codes and the slot's scale per chunk; the
    // codes go to LDS as bf16, each token's scales beside the tiles)
    Loaded8<Q8> kr[CPT], vr[CPT];
    auto load = [&](uint32_t tb) {
#pragma unroll
        for (uint32_t e = 0; e < CPT; ++e) {
            const uint32_t ch = threadIdx.x + kAttnThreads * e;
            const uint32_t jt = ch / (D / 8), dc = ch % (D / 8);
            const uint32_t j = min32(tb + jt, n - 1);
            const uint32_t pj = udiv32(j, a.div_page);
            if constexpr (Q8) {
                const uint64_t slot = pages[pj] + (j - pj * P);
                const uint64_t off = slot * slot_bytes + head_off + 8 * dc;
                kr[e] = Raw8{ld8<false>(a.k_pool + off), a.k_scales[slot]};
                vr[e] = Raw8{ld8<false>(a.v_pool + off), a.v_scales[slot]};
            } else {
                const uint64_t off = pages[pj] + (uint64_t)(j - pj * P) * slot_bytes +
                                     head_off + 16 * dc;
                kr[e] = ld16<false>(a.k_pool + off);
                vr[e] = ld16<false>(a.v_pool + off);
            }
        }
    };
    load(0);
    uint32_t stage = 0;
    for (uint32_t tb = 0; tb < n; tb += kMfmaTile) {
        unsigned char *kt = region + (2 * stage) * WL, *vt = region + (2 * stage + 1) * WL;
#pragma unroll
        for (uint32_t e = 0; e < CPT; ++e) {
            const uint32_t ch = threadIdx.x + kAttnThreads * e;
            const uint32_t jt = ch / (D / 8), dc = ch % (D / 8);
            *reinterpret_cast<u32x4 *>(kt + jt * VRB + 16 * dc) = bits8(kr[e]);
            *reinterpret_cast<u32x4 *>(vt + jt * VRB + 16 * dc) = bits8(vr[e]);
            if (Q8 && dc == 0) {
                scl[(2 * stage) * kMfmaTile + jt] = row_scale(kr[e]);
                scl[(2 * stage + 1) * kMfmaTile + jt] = row_scale(vr[e]);
            }
        }
        // the stage is written; every wave finished the tile that last used
        // the other stage before it reached this barrier
        __syncthreads();
        if (tb + kMfmaTile < n)
            load(tb + kMfmaTile);
        lds_tile<ET, D, Q8>(a, kt, vt, scl + (2 * stage) * kMfmaTile,
                            scl + (2 * stage + 1) * kMfmaTile, pt, tb, n, qa, m, l, o);
        stage ^= 1;
    }

    // row 4 grp + i: the partial result of chunk c goes to unit slot c of its
    // sequence; a sequence whose only unit this is gets its output directly
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t seq, qi;
        if (!row_seq(4 * grp + i, seq, qi))
            continue;
        const uint32_t u0 = seq ? a.unit_end[seq - 1] : 0, u1 = a.unit_end[seq];
        if (u0 + c >= u1)
            continue;  // units capped (total_tokens below the counts): no slot
        const uint64_t hq = (uint64_t)h * G + qi;
        if (u1 - u0 == 1) {
            float *dst = a.out + ((uint64_t)seq * Hq + hq) * D + c16;
#pragma unroll
            for (uint32_t db = 0; db < DB; ++db)
                dst[16 * db] = o[db][i] / l[i];
        } else {
            const uint64_t idx = (uint64_t)(u0 + c) * Hq + hq;
            float *dst = a.part_acc + idx * D + c16;
#pragma unroll
            for (uint32_t db = 0; db < DB; ++db)
                dst[16 * db] = o[db][i];
            if (c16 == 0) {
                a.part_ml[2 * idx] = m[i];
                a.part_ml[2 * idx + 1] = l[i];
            }
        }
    }
}

// Which matrix-core grids take their head groups interleaved in blockIdx.x
// (bit 0: grids without the shared-prefix pass; bit 1: int8 grids with it).
// Measured on MI355X, cold caches, against head groups in blockIdx.y: decode
// batch G = 4 193.3 -> 189.4 us, G = 8 205.4 -> 201.9 us, int8 pools at G = 4
// 122.3 -> 114.5 us; prefix batch over int8 pools 91.4 -> 84.4 us, but over
// 16-bit pools at G = 8 108.3 -> 118.8 us (so not there). The vector kernel
// (two head groups of 16 heads on the decode batch) measured no change.
#ifndef HP_ATTN_HG_INTERLEAVE
#define HP_ATTN_HG_INTERLEAVE 3
#endif
// Waves per SIMD the matrix-core kernel is built for when its grid carries
// the shared-prefix pass (16-bit pools). Measured on MI355X, prefix batch:
// three waves (a few registers spilled) against two, G = 4: 100.4 -> 95.3 us,
// G = 8: 121.3 -> 110.0 us; the same bound on the streamed decode batch lost
// 5 % (192.3 -> 202.3 us at G = 4), so only the grids with the pass take it.
#ifndef HP_ATTN_SHARED_WAVES
#define HP_ATTN_SHARED_WAVES 3
#endif

// R: accumulator rows per lane that hold query heads (1 for G <= 4, 2 for
// G <= 8, else 4). Q8: int8 pools with per-slot scales (ET is then BF16).
// SH: the grid carries the shared-prefix pass (a.shared).
template <typename ET, typename IdxT, int D, bool NT, int R, bool Q8, bool SH>
__global__ __launch_bounds__(kAttnThreads, Q8 ? 2 : (SH ? HP_ATTN_SHARED_WAVES : 1))
void attention_mfma_kernel(AArgs a) {
#pragma clang fp contract(off)
    using M = Mma<ET>;
    using V8 = typename M::V8;
    constexpr uint32_t KK = D / 32;  // MFMAs per 16-token score block
    constexpr uint32_t DB = D / 16;  // 16-column blocks of the output
    constexpr uint32_t VRB = v_row_bytes<D>();
    extern __shared__ __align__(16) unsigned char lds[];
    const uint32_t S = a.num_seqs;
    const uint32_t by = a.hg_il ? blockIdx.x % a.hg_il : blockIdx.y;
    uint32_t g = a.hg_il ? blockIdx.x / a.hg_il : blockIdx.x;
    if constexpr (SH) {
        // the shared-prefix work items come first, so that their reads (mostly
        // served by the caches) overlap the units' HBM reads
        // (one kv head per workgroup: kMfmaWaves workgroups per item and
        // grid row)
        const uint32_t nw = uni(*a.nwork) * kMfmaWaves;
        if (g < nw) {
            const uint32_t h = by * kMfmaWaves + g % kMfmaWaves;
            if (h < a.num_kv_heads)
                shared_item<ET, IdxT, D, Q8>(a, g / kMfmaWaves, h, lds);
            return;
        }
        g -= nw;
    }
    const size_t ue_bytes = a.fused ? ((4 * (size_t)S + 15) & ~(size_t)15) : 0;
    uint32_t *ue_lds = reinterpret_cast<uint32_t *>(lds);
    uint64_t *pages = reinterpret_cast<uint64_t *>(lds + ue_bytes);
    const uint32_t *unit_end = a.unit_end;
    if (a.fused) {
        unit_scan_lds<IdxT>(a.seq_lens, S, a.unit_tokens, a.cap_units, ue_lds);
        unit_end = ue_lds;
    }

    const uint32_t total = uni(unit_end[S - 1]);
    const uint32_t Hq = a.num_q_heads, Hkv = a.num_kv_heads, P = a.page_size, G = a.group;
    const uint32_t gz = blockIdx.z * kMfmaRows;  // first query head of this chunk in the group
    if (g >= total) {
        // spare workgroups: workgroup total + s writes the zeros of sequence s
        // when it has no token
        const uint32_t se = g - total;
        if (se >= S || blockIdx.z != 0 || ld_idx<IdxT>(a.seq_lens, se) != 0)
            return;
        const uint32_t h0 = by * kMfmaWaves;
        const uint32_t nq = (min32(Hkv, h0 + kMfmaWaves) - h0) * G;
        float *o = a.out + ((uint64_t)se * Hq + (uint64_t)h0 * G) * D;
        for (uint32_t e = threadIdx.x; e < nq * D; e += kAttnThreads)
            o[e] = 0.0f;
        return;
    }
    uint32_t s;
    if (a.fused) {
        uint32_t lo = 0, hi = S - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (ue_lds[mid] > g)
                hi = mid;
            else
                lo = mid + 1;
        }
        s = uni(lo);
    } else {
        s = uni(a.unit_seq[g]);
    }
    const uint32_t u0 = s ? uni(unit_end[s - 1]) : 0;
    const uint64_t L = uni64(ld_idx<IdxT>(a.seq_lens, s));
    const uint64_t sp0 = uni64(ld_idx<IdxT>(a.seq_ptr, s));
    // The sequence's units: with the shared pass, first its shared chunks
    // (computed by the shared items), then ns units over the rest; the rest's
    // pages are split evenly among those (each holds at most unit_pages, as
    // ns = ceil(rest / unit_tokens), and at least one, as unit_tokens >= P).
    uint64_t sh_tokens = 0;
    uint32_t k = g - u0;
    if constexpr (SH) {
        const uint32_t sh = uni(a.pre_pages[s]);
        const uint32_t nch = (sh + a.chunk_pages - 1) / a.chunk_pages;
        if (k < nch)
            return;
        k -= nch;
        sh_tokens = (uint64_t)sh * P;
    }
    if (sh_tokens >= L)
        return;  // only when total_tokens disagrees with the counts: read nothing
    const uint64_t rest = L - sh_tokens;
    const uint64_t ns = (rest + a.unit_tokens - 1) / a.unit_tokens;
    const uint64_t rest_pages = (rest + P - 1) / P;
    const uint64_t p_begin = k * rest_pages / ns, p_end = (k + 1) * rest_pages / ns;
    const uint64_t t0 = sh_tokens + p_begin * P;
    if (k >= ns || t0 >= L)
        return;  // only when total_tokens disagrees with the counts: read nothing
    const uint32_t n = (uint32_t)min64(L - t0, (p_end - p_begin) * P);
    const uint64_t pg0 = t0 / P;
    const uint32_t npg = udiv32(n + P - 1, a.div_page);
    // byte offsets of the pages (int8 pools: their first slots)
    const uint64_t page_mul = Q8 ? (uint64_t)P : (uint64_t)P * Hkv * D * 2;
    for (uint32_t i = threadIdx.x; i < npg; i += kAttnThreads)
        pages[i] = ld_idx<IdxT>(a.block_table, sp0 + pg0 + i) * page_mul;
    __syncthreads();

    const uint32_t wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const uint32_t h = by * kMfmaWaves + wave;
    if (h >= Hkv)
        return;  // no barrier follows
    unsigned char *vt = lds + ue_bytes + a.pg_area + wave * mfma_wave_lds<D>();
    float *pt = reinterpret_cast<float *>(vt + kMfmaTile * VRB);
    const uint32_t c16 = lane & 15, grp = lane >> 4;
    // Q as the A operand of the score product: row c16 is query head
    // gz + row_head(c16) of this kv head (zero past G); lane group grp holds
    // dims 32 kk + 8 grp.
    V8 qa[KK];
    {
        const uint32_t qh = gz + row_head(c16);
        const bool qrow = qh < G;
        const uint64_t qo = (((uint64_t)s * Hq + (uint64_t)h * G + min32(qh, G - 1)) * D +
                             8 * grp) * 2;
#pragma unroll
        for (uint32_t kk = 0; kk < KK; ++kk) {
            u32x4 v = ld16<false>(a.q + qo + kk * 64);
            if (!qrow)
                v = u32x4(0);
            qa[kk] = __builtin_bit_cast(V8, v);
        }
    }
    float m[4], l[4];
    f32x4 o[DB];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m[i] = -__builtin_inff();
        l[i] = 0.0f;
    }
#pragma unroll
    for (uint32_t db = 0; db < DB; ++db)
        o[db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    mfma_span<ET, D, NT, R, Q8>(a, pages, n, h, qa, vt, pt, m, l, o);

    // rows 4 grp + i: query head gz + 4 i + grp of kv head h, column 16 db + c16
    const uint32_t units = uni(unit_end[s]) - u0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const uint32_t qi = gz + 4 * i + grp;
        if (qi >= G)
            continue;
        const uint64_t hq = (uint64_t)h * G + qi;
        if (units == 1) {
            float *dst = a.out + ((uint64_t)s * Hq + hq) * D + c16;
#pragma unroll
            for (uint32_t db = 0; db < DB; ++db)
                dst[16 * db] = o[db][i] / l[i];
        } else {
            const uint64_t idx = (uint64_t)g * Hq + hq;
            float *dst = a.part_acc + idx * D + c16;
#pragma unroll
            for (uint32_t db = 0; db < DB; ++db)
                dst[16 * db] = o[db][i];
            if (c16 == 0) {
                a.part_ml[2 * idx] = m[i];
                a.part_ml[2 * idx + 1] = l[i];
            }
        }
    }
}

struct PlanArgs {
    const void *block_table, *seq_ptr, *seq_lens;
    uint32_t num_seqs, page_size, unit_tokens, chunk_pages, min_pages, seqs_per_block;
    uint32_t cap_units, cap_work;
    uint32_t *unit_end, *unit_seq, *pre_pages, *run_of, *run_first, *run_c;
    uint32_t *work_seq0, *work_chunk, *nwork;
};

// Exclusive scan of v over the workgroup (one value per thread); *total gets
// the sum. Every thread calls it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *total) {
    __shared__ uint32_t wave_sum[kAttnThreads / 64];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= (uint32_t)o)
            incl += y;
    }
    if (lane == 63)
        wave_sum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (uint32_t k = 0; k < kAttnThreads / 64; ++k) {
        before += k < wave ? wave_sum[k] : 0;
        all += wave_sum[k];
    }
    __syncthreads();  // wave_sum may be reused by the next call
    *total = all;
    return before + incl - v;
}

// Leading pages that sequence s > 0 has in common with sequence s - 1: equal
// page IDs at the same positions of the two slices, counting only pages that
// both sequences fill (and at most kMaxSharedPages), into pre_pages[s]; 0
// for s = 0. One wave per sequence compares 64 x kLcpPerLane positions per
// step.
constexpr uint32_t kMaxSharedPages = 8192;
constexpr uint32_t kLcpPerLane = 4;

template <typename IdxT>
__global__ __launch_bounds__(kAttnThreads) void attention_lcp_kernel(PlanArgs p) {
    const uint32_t s = blockIdx.x * (kAttnThreads / 64) + (threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    if (s >= p.num_seqs)
        return;
    uint64_t lcp = 0;
    if (s > 0) {
        const uint32_t P = p.page_size;
        const uint64_t a0 = uni64(ld_idx<IdxT>(p.seq_ptr, s - 1));
        const uint64_t a1 = uni64(ld_idx<IdxT>(p.seq_ptr, s));
        const uint64_t b1 = uni64(ld_idx<IdxT>(p.seq_ptr, s + 1));
        uint64_t lim = uni64(ld_idx<IdxT>(p.seq_lens, s - 1)) / P;
        lim = min64(lim, uni64(ld_idx<IdxT>(p.seq_lens, s)) / P);
        lim = min64(lim, min64(a1 - a0, b1 - a1));
        lim = min64(lim, kMaxSharedPages);
        lcp = lim;
        for (uint64_t base = 0; base < lim; base += 64 * kLcpPerLane) {
            uint64_t x[kLcpPerLane], y[kLcpPerLane];
#pragma unroll
            for (uint32_t k = 0; k < kLcpPerLane; ++k) {
                const uint64_t j = base + 64 * k + lane;
                x[k] = j < lim ? ld_idx<IdxT>(p.block_table, a0 + j) : 0;
                y[k] = j < lim ? ld_idx<IdxT>(p.block_table, a1 + j) : 0;
            }
            uint64_t first = ~0ull;
#pragma unroll
            for (uint32_t k = kLcpPerLane; k-- > 0;) {
                const uint64_t mask = __ballot(x[k] != y[k]);
                if (mask)
                    first = base + 64 * k + (uint64_t)(__ffsll((long long)mask) - 1);
            }
            if (first != ~0ull) {
                lcp = first;
                break;
            }
        }
    }
    if (lane == 0)
        p.pre_pages[s] = (uint32_t)lcp;
}

// The shared-prefix plan, one workgroup, after attention_lcp_kernel: runs of
// sequences that share leading pages (a run starts where a sequence's count
// of leading pages in common with its predecessor is below min_pages), each
// sequence's shared pages (its run's smallest count; 0 for a run of one), the
// units (shared chunks, then units over the rest) with unit_end and the unit
// -> sequence map, and the shared pass's work items (a run block of
// seqs_per_block sequences times the chunks of its shared pages).
// Up to kPlanLdsSeqs sequences the per-sequence arrays live in LDS while the
// plan runs (each pass then costs LDS latency, not a global round trip) and
// run_of and pre_pages are copied out at the end; beyond it they stay in the
// workspace.
constexpr uint32_t kPlanLdsSeqs = 2048;

template <typename IdxT>
__global__ __launch_bounds__(kAttnThreads) void attention_prefix_plan_kernel(PlanArgs p) {
    __shared__ uint32_t l_run[kPlanLdsSeqs], l_first[kPlanLdsSeqs], l_c[kPlanLdsSeqs],
        l_pre[kPlanLdsSeqs], l_ue[kPlanLdsSeqs];
    const uint32_t S = p.num_seqs, P = p.page_size;
    const bool in_lds = S <= kPlanLdsSeqs;
    uint32_t *run_of = in_lds ? l_run : p.run_of, *run_first = in_lds ? l_first : p.run_first;
    uint32_t *run_c = in_lds ? l_c : p.run_c, *pre = in_lds ? l_pre : p.pre_pages;
    uint32_t *unit_end = in_lds ? l_ue : p.unit_end;
    // 1. run ids and firsts from the common leading pages
    uint32_t runs = 0;
    for (uint32_t base = 0; base < S; base += kAttnThreads) {
        const uint32_t s = base + threadIdx.x;
        uint32_t lcp = 0, start = 0;
        if (s < S) {
            lcp = p.pre_pages[s];
            start = (s == 0 || lcp < p.min_pages) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t before = block_exclusive_scan(start, &tot);
        if (s < S) {
            const uint32_t rid = runs + before + start - 1;
            run_of[s] = rid;
            pre[s] = lcp;
            if (start)
                run_first[rid] = s;
        }
        runs += tot;
    }
    __syncthreads();
    for (uint32_t r = threadIdx.x; r < runs; r += kAttnThreads)
        run_c[r] = ~0u;
    __syncthreads();
    // 2. a run's shared pages: the smallest common count of its members
    for (uint32_t s = threadIdx.x; s < S; s += kAttnThreads) {
        const uint32_t rid = run_of[s];
        if (run_first[rid] != s)
            atomicMin(&run_c[rid], pre[s]);
    }
    __syncthreads();
    for (uint32_t s = threadIdx.x; s < S; s += kAttnThreads) {
        const uint32_t cr = __hip_atomic_load(&run_c[run_of[s]], __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        pre[s] = cr == ~0u ? 0u : cr;
    }
    __syncthreads();
    // 3. units and work items
    uint32_t units = 0, work = 0;
    for (uint32_t base = 0; base < S; base += kAttnThreads) {
        const uint32_t s = base + threadIdx.x;
        uint32_t nu = 0, nw = 0, nch = 0;
        if (s < S) {
            const uint32_t sh = pre[s];
            nch = (sh + p.chunk_pages - 1) / p.chunk_pages;
            const uint64_t rest = ld_idx<IdxT>(p.seq_lens, s) - (uint64_t)sh * P;
            nu = nch + (uint32_t)(rest / p.unit_tokens + (rest % p.unit_tokens != 0));
            const uint32_t pos = s - run_first[run_of[s]];
            if (sh && pos % p.seqs_per_block == 0)
                nw = nch;
        }
        uint32_t tu, tw;
        const uint32_t ub = block_exclusive_scan(nu, &tu);
        const uint32_t wb = block_exclusive_scan(nw, &tw);
        if (s < S) {
            const uint32_t ue = min32(units + ub + nu, p.cap_units);
            unit_end[s] = ue;
            if (in_lds) {
                p.unit_end[s] = ue;
                p.run_of[s] = run_of[s];
                p.pre_pages[s] = pre[s];
            }
            for (uint32_t k = 0; k < nw && work + wb + k < p.cap_work; ++k) {
                p.work_seq0[work + wb + k] = s;
                p.work_chunk[work + wb + k] = k;
            }
        }
        units += tu;
        work += tw;
    }
    __syncthreads();
    if (threadIdx.x == 0)
        *p.nwork = min32(work, p.cap_work);
    // 4. the unit -> sequence map (this workgroup's unit_end stores are
    // visible to it after the barrier)
    const uint32_t total = min32(units, p.cap_units);
    for (uint32_t u = threadIdx.x; u < total; u += kAttnThreads) {
        uint32_t lo = 0, hi = S - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (unit_end[mid] > u)
                hi = mid;
            else
                lo = mid + 1;
        }
        p.unit_seq[u] = lo;
    }
}

// Running unit count per sequence, unit_end[s] = sum over s' <= s of
// ceil(L_s' / U) (capped at the workspace's unit capacity), and the sequence
// of every unit, unit_seq[u]. One workgroup.
template <typename IdxT>
__global__ __launch_bounds__(kAttnThreads) void attention_plan_kernel(const void *seq_lens,
                                                                      uint32_t S, uint32_t U,
                                                                      uint32_t cap,
                                                                      uint32_t *unit_end,
                                                                      uint32_t *unit_seq) {
    __shared__ uint64_t wave_sum[kAttnThreads / 64];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t running = 0;
    for (uint32_t base = 0; base < S; base += kAttnThreads) {
        const uint32_t i = base + threadIdx.x;
        uint64_t v = 0;
        if (i < S) {
            const uint64_t len = ld_idx<IdxT>(seq_lens, i);
            v = len / U + (len % U != 0);
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint64_t y = __shfl_up(v, o, 64);
            if (lane >= (uint32_t)o)
                v += y;
        }
        if (lane == 63)
            wave_sum[wave] = v;
        __syncthreads();
        uint64_t before = running;
        for (uint32_t w = 0; w < wave; ++w)
            before += wave_sum[w];
        if (i < S)
            unit_end[i] = (uint32_t)min64(before + v, cap);
        for (uint32_t w = 0; w < kAttnThreads / 64; ++w)
            running += wave_sum[w];
        __syncthreads();
    }
    // unit -> sequence map: the workgroup's own unit_end stores are visible to
    // it after the barrier above
    const uint32_t total = S ? unit_end[S - 1] : 0;
    for (uint32_t u = threadIdx.x; u < total; u += kAttnThreads) {
        uint32_t lo = 0, hi = S - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (unit_end[mid] > u)
                hi = mid;
            else
                lo = mid + 1;
        }
        unit_seq[u] = lo;
    }
}

struct CArgs {
    const uint32_t *unit_end;  // null: count the units here (fused)
    const void *seq_lens;
    const float *part_ml, *part_acc;
    float *out;
    uint32_t num_q_heads, head_dim, unit_tokens, cap_units;
    Div div_d;
};

// [first, end) units of sequence s, counted by the workgroup from the token
// counts (a block sum over the sequences before s) when there is no plan.
template <typename IdxT>
__device__ __forceinline__ void seq_units(const CArgs &c, uint32_t s, uint32_t &u0, uint32_t &u1) {
    if (c.unit_end) {
        u0 = s ? c.unit_end[s - 1] : 0;
        u1 = c.unit_end[s];
        return;
    }
    __shared__ uint32_t wave_sum[kAttnThreads / 64];
    uint32_t v = 0;
    for (uint32_t i = threadIdx.x; i < s; i += kAttnThreads)
        v += units_of_seq<IdxT>(c.seq_lens, i, c.unit_tokens);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0)
        wave_sum[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t before = 0;
    for (uint32_t w = 0; w < kAttnThreads / 64; ++w)
        before += wave_sum[w];
    u0 = min32(before, c.cap_units);
    u1 = min32(before + units_of_seq<IdxT>(c.seq_lens, s, c.unit_tokens), c.cap_units);
}

// out[s][hq][d] of a sequence held by several units: the units' partial
// results merged with max-shifted weights, then divided. One pass over the
// units, B at a time so that their loads are in flight together.
template <uint32_t B>
__device__ __forceinline__ void combine_units(const CArgs &c, uint32_t s, uint32_t u0, uint32_t u1,
                                              uint32_t i) {
    const uint32_t Hq = c.num_q_heads, D = c.head_dim;
    const uint32_t hq = udiv32(i, c.div_d), d = i - hq * D;
    float M = -__builtin_inff(), lsum = 0.0f, num[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (uint32_t ub = u0; ub < u1; ub += B) {
        float mv[B], lv[B];
        u32x4 av[B];
#pragma unroll
        for (uint32_t k = 0; k < B; ++k) {
            const uint32_t u = ub + k < u1 ? ub + k : u1 - 1;  // repeats get weight 0 below
            const uint64_t idx = (uint64_t)u * Hq + hq;
            mv[k] = c.part_ml[2 * idx];
            lv[k] = c.part_ml[2 * idx + 1];
            av[k] = *reinterpret_cast<const u32x4 *>(c.part_acc + idx * D + d);
        }
        float Mn = M;
#pragma unroll
        for (uint32_t k = 0; k < B; ++k)
            Mn = __builtin_fmaxf(Mn, mv[k]);
        const float cs = exp2_hw(M - Mn);  // M = -inf on the first batch: 0
        lsum *= cs;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            num[e] *= cs;
#pragma unroll
        for (uint32_t k = 0; k < B; ++k) {
            const float w = ub + k < u1 ? exp2_hw(mv[k] - Mn) : 0.0f;
            float a4[4];
            __builtin_memcpy(a4, &av[k], 16);
            lsum = __builtin_fmaf(lv[k], w, lsum);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                num[e] = __builtin_fmaf(a4[e], w, num[e]);
        }
        M = Mn;
    }
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = num[e] / lsum;
    u32x4 ov;
    __builtin_memcpy(&ov, o, 16);
    *reinterpret_cast<u32x4 *>(c.out + (uint64_t)s * Hq * D + i) = ov;
}

// Sequences of zero or one unit were written by the attention kernel. The
// batch of units loaded together follows the sequence's unit count (the
// same merge in the same order; only the loads of repeated units differ).
template <typename IdxT>
__global__ __launch_bounds__(kAttnThreads) void attention_combine_kernel(CArgs c) {
    const uint32_t s = blockIdx.x;
    uint32_t u0, u1;
    seq_units<IdxT>(c, s, u0, u1);
    if (u1 - u0 < 2)
        return;
    // each thread: 4 consecutive outputs of one query head (head_dim % 8 == 0)
    const uint32_t i = (blockIdx.y * kAttnThreads + threadIdx.x) * 4;
    if (i >= c.num_q_heads * c.head_dim)
        return;
    const uint32_t n = u1 - u0;
    if (n <= 4)
        combine_units<4>(c, s, u0, u1, i);
    else if (n <= 8)
        combine_units<8>(c, s, u0, u1, i);
    else
        combine_units<16>(c, s, u0, u1, i);
}

// ---- host side ----------------------------------------------------------------

// Query-head slots per lane group for G query heads per kv head.
uint32_t group_slots(uint32_t G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8; }

// Codes per lane of the vector kernel over int8 pools: 16 (one 16-byte load,
// the bytes in flight of a 16-bit pool's lane) for one or two query heads
// per kv head and head_dim >= 16; else 8 (the accumulators of 16 elements
// for four or eight query-head slots would not fit in registers).
uint32_t q8_lane_codes(uint32_t D, uint32_t G) {
    return D >= 16 && group_slots(G) <= 2 ? 16 : 8;
}

// Grouped query heads with head_dim 64 or 128 take the matrix-core kernel
// from three query heads per kv head, and at two when the loads stream (each
// page read once, so HBM bounds the call). Measured on MI355X against the
// vector kernel: 1.4x faster at G = 4 and 1.9x at G = 8 (prefix batch); at
// G = 2, 12 % faster on the streamed decode batch but 8 % slower on the
// prefix batch, whose shared pages come from the caches.
#ifndef HP_ATTN_MFMA_MIN_GROUP
#define HP_ATTN_MFMA_MIN_GROUP 3
#endif
// Workgroups aimed at with one query head per kv head and cached loads.
// Measured on MI355X (prefix batch, 8 kv heads): 4,096 runs 16 % faster than
// 1,024; with streaming loads (decode batch) 1,024 stays best (4,096: 14 %
// slower).
#ifndef HP_ATTN_TARGET_GROUPS_MHA_CACHED
#define HP_ATTN_TARGET_GROUPS_MHA_CACHED 4096
#endif
constexpr uint64_t kAttnTargetGroupsMhaCached = HP_ATTN_TARGET_GROUPS_MHA_CACHED;

bool attention_mfma(uint32_t G, uint32_t D, bool stream) {
    const uint32_t min_group = stream && HP_ATTN_MFMA_MIN_GROUP > 2 ? 2 : HP_ATTN_MFMA_MIN_GROUP;
    return G >= min_group && (D == 64 || D == 128);
}

template <typename ET, typename IdxT, int D, int R, bool Q8>
hipError_t launch_attention_mfma(const AArgs &a, const AttentionShape &sh, bool nt,
                                 hipStream_t stream) {
    // shared work items (at most cap_work), units, then one spare per sequence
    const uint64_t gx = sh.cap_units + a.num_seqs + (a.shared ? kMfmaWaves * sh.cap_work : 0);
    const uint32_t gz = (a.group + kMfmaRows - 1) / kMfmaRows;
    // Head groups interleaved (the head groups of one work index neighbours
    // in the dispatch order, so that their pieces of each token row are read
    // together) on the grids where it measured faster.
    AArgs b = a;
    const uint32_t il_bit = a.shared ? (Q8 ? 2u : 0u) : 1u;
    const bool il = (HP_ATTN_HG_INTERLEAVE & il_bit) && sh.head_groups > 1 &&
                    gx * sh.head_groups < (1ull << 31);
    b.hg_il = il ? sh.head_groups : 0;
    const dim3 grid = il ? dim3((uint32_t)(gx * sh.head_groups), 1, gz)
                         : dim3((uint32_t)gx, sh.head_groups, gz);
    // (int8 pools: the shared pass keeps two stages of K and V scales too)
    const size_t lds = (a.fused ? ((4 * (size_t)a.num_seqs + 15) & ~(size_t)15) : 0) +
                       a.pg_area + kMfmaWaves * mfma_wave_lds<D>() +
                       (Q8 ? 2 * 2 * kMfmaTile * sizeof(float) : 0);
    // (the shared pass streams its units: nt is set whenever a.shared is)
    if (a.shared)
        hipLaunchKernelGGL((attention_mfma_kernel<ET, IdxT, D, true, R, Q8, true>), grid,
                           dim3(kAttnThreads), lds, stream, b);
    else if (nt)
        hipLaunchKernelGGL((attention_mfma_kernel<ET, IdxT, D, true, R, Q8, false>), grid,
                           dim3(kAttnThreads), lds, stream, b);
    else
        hipLaunchKernelGGL((attention_mfma_kernel<ET, IdxT, D, false, R, Q8, false>), grid,
                           dim3(kAttnThreads), lds, stream, b);
    return hipGetLastError();
}

template <typename ET, typename IdxT, int D, bool Q8>
hipError_t launch_mfma_r(const AArgs &a, const AttentionShape &sh, uint32_t G, bool nt,
                         hipStream_t st) {
    if (G <= 4)
        return launch_attention_mfma<ET, IdxT, D, 1, Q8>(a, sh, nt, st);
    if (G <= 8)
        return launch_attention_mfma<ET, IdxT, D, 2, Q8>(a, sh, nt, st);
    return launch_attention_mfma<ET, IdxT, D, 4, Q8>(a, sh, nt, st);
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

template <typename ET, typename IdxT, int LPH, int GT, bool Q8, int EPL>
hipError_t launch_attention_t(const AArgs &a, const AttentionShape &sh, bool nt,
                              hipStream_t stream) {
    const dim3 grid((uint32_t)(sh.cap_units + a.num_seqs), sh.head_groups,
                    (a.group + GT - 1) / GT);
    const uint32_t ng = kAttnThreads / LPH;
    const size_t lds = (a.fused ? ((4 * (size_t)a.num_seqs + 15) & ~(size_t)15) : 0) +
                       8 * (size_t)a.unit_pages +
                       (sh.token_lanes > 1 ? 4 * (size_t)ng * (2 + LPH * EPL) : 0);
    if (nt)
        hipLaunchKernelGGL((attention_kernel<ET, IdxT, LPH, GT, true, Q8, EPL>), grid,
                           dim3(kAttnThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((attention_kernel<ET, IdxT, LPH, GT, false, Q8, EPL>), grid,
                           dim3(kAttnThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename ET, typename IdxT, int LPH, bool Q8, int EPL>
hipError_t launch_attention_g(const AArgs &a, const AttentionShape &sh, uint32_t G, bool nt,
                              hipStream_t st) {
    if constexpr (EPL == 16) {  // one or two query heads per kv head
        if (group_slots(G) == 1)
            return launch_attention_t<ET, IdxT, LPH, 1, Q8, 16>(a, sh, nt, st);
        return launch_attention_t<ET, IdxT, LPH, 2, Q8, 16>(a, sh, nt, st);
    }
    switch (group_slots(G)) {
    case 1: return launch_attention_t<ET, IdxT, LPH, 1, Q8, EPL>(a, sh, nt, st);
    case 2: return launch_attention_t<ET, IdxT, LPH, 2, Q8, EPL>(a, sh, nt, st);
    case 4: return launch_attention_t<ET, IdxT, LPH, 4, Q8, EPL>(a, sh, nt, st);
    default: return launch_attention_t<ET, IdxT, LPH, 8, Q8, EPL>(a, sh, nt, st);
    }
}

template <typename ET, typename IdxT, bool Q8>
hipError_t launch_attention_d(const AArgs &a, const AttentionShape &sh, uint32_t G, bool nt,
                              hipStream_t st) {
    if constexpr (Q8) {
        if (q8_lane_codes(a.head_dim, G) == 16) {
            switch (a.head_dim) {
            case 16: return launch_attention_g<ET, IdxT, 1, Q8, 16>(a, sh, G, nt, st);
            case 32: return launch_attention_g<ET, IdxT, 2, Q8, 16>(a, sh, G, nt, st);
            case 64: return launch_attention_g<ET, IdxT, 4, Q8, 16>(a, sh, G, nt, st);
            case 128: return launch_attention_g<ET, IdxT, 8, Q8, 16>(a, sh, G, nt, st);
            default: return launch_attention_g<ET, IdxT, 16, Q8, 16>(a, sh, G, nt, st);
            }
        }
    }
    switch (a.head_dim) {
    case 8: return launch_attention_g<ET, IdxT, 1, Q8, 8>(a, sh, G, nt, st);
    case 16: return launch_attention_g<ET, IdxT, 2, Q8, 8>(a, sh, G, nt, st);
    case 32: return launch_attention_g<ET, IdxT, 4, Q8, 8>(a, sh, G, nt, st);
    case 64: return launch_attention_g<ET, IdxT, 8, Q8, 8>(a, sh, G, nt, st);
    case 128: return launch_attention_g<ET, IdxT, 16, Q8, 8>(a, sh, G, nt, st);
    default: return launch_attention_g<ET, IdxT, 32, Q8, 8>(a, sh, G, nt, st);
    }
}

// Q8: int8 pools with per-slot scales, computed as bf16 (ET = BF16).
template <typename ET, bool Q8>
hipError_t launch_attention_i(const AArgs &a, const AttentionShape &sh, uint32_t G, bool idx64,
                              bool nt, hipStream_t st) {
    static_assert(!Q8 || ET::bf16, "int8 pools dequantise to bf16");
    if (attention_mfma(G, a.head_dim, nt)) {
        if (a.head_dim == 64)
            return idx64 ? launch_mfma_r<ET, uint64_t, 64, Q8>(a, sh, G, nt, st)
                         : launch_mfma_r<ET, uint32_t, 64, Q8>(a, sh, G, nt, st);
        return idx64 ? launch_mfma_r<ET, uint64_t, 128, Q8>(a, sh, G, nt, st)
                     : launch_mfma_r<ET, uint32_t, 128, Q8>(a, sh, G, nt, st);
    }
    return idx64 ? launch_attention_d<ET, uint64_t, Q8>(a, sh, G, nt, st)
                 : launch_attention_d<ET, uint32_t, Q8>(a, sh, G, nt, st);
}

struct WsLayout {
    uint64_t unit_end, unit_seq, ml, acc, end;
    // the prefix plan's arrays (shared-prefix pass only)
    uint64_t pre_pages, run_of, run_first, run_c, work_seq0, work_chunk, nwork;
};

WsLayout ws_layout(uint64_t S, uint64_t Hq, uint64_t D, const AttentionShape &sh) {
    const uint64_t cap = sh.cap_units;
    const uint64_t sS = sh.shared ? S : 0, sW = sh.shared ? sh.cap_work : 0;
    WsLayout w;
    w.unit_end = 256;  // the validator's words come first
    w.unit_seq = w.unit_end + align256(4 * S);
    w.pre_pages = w.unit_seq + align256(4 * cap);
    w.run_of = w.pre_pages + align256(4 * sS);
    w.run_first = w.run_of + align256(4 * sS);
    w.run_c = w.run_first + align256(4 * sS);
    w.work_seq0 = w.run_c + align256(4 * sS);
    w.work_chunk = w.work_seq0 + align256(4 * sW);
    w.nwork = w.work_chunk + align256(4 * sW);
    w.ml = w.nwork + (sh.shared ? 256 : 0);
    w.acc = w.ml + align256(8 * cap * Hq);
    w.end = w.acc + align256(4 * cap * Hq * D);
    return w;
}

} // namespace

AttentionShape attention_shape(uint64_t num_seqs, uint64_t total_tokens, uint32_t page_size,
                               uint32_t num_kv_heads, uint32_t head_dim, uint32_t num_q_heads,
                               bool stream_loads, bool q8) {
    AttentionShape sh;
    const uint32_t G = num_q_heads / num_kv_heads;
    const bool mfma = attention_mfma(G, head_dim, stream_loads);
    if (mfma) {
        // one wave per kv head, four kv heads per workgroup
        sh.heads_per_group = kMfmaWaves;
        sh.token_lanes = 1;
    } else {
        // lanes per head row: 8 elements each, or 16 int8 codes
        const uint32_t lph = head_dim / (q8 ? q8_lane_codes(head_dim, G) : 8);
        const uint32_t ng = kAttnThreads / lph;
        sh.heads_per_group = num_kv_heads < ng ? num_kv_heads : ng;
        sh.token_lanes = ng / sh.heads_per_group;
    }
    sh.head_groups = (num_kv_heads + sh.heads_per_group - 1) / sh.heads_per_group;
    // Pages to visit (at most), spread over about kAttnTargetGroups workgroups.
    const uint64_t pages = total_tokens / page_size + num_seqs;
    // one query head per kv head: few, long units when the loads stream
    // (HBM bounds the call), more and shorter ones when they are served from
    // the caches; grouped heads (more arithmetic per byte) spread over more
    // workgroups
    const uint64_t target = num_q_heads != num_kv_heads
                                ? (stream_loads ? kAttnTargetGroupsGqaStream : kAttnTargetGroupsGqa)
                            : stream_loads              ? kAttnTargetGroupsMha
                                                        : kAttnTargetGroupsMhaCached;
    uint64_t upages = (pages * sh.head_groups + target - 1) / target;
    // each unit writes (D + 2) floats per query head it covers: keep that a
    // small share of the unit's K/V bytes (2 D per token and kv head)
    uint64_t min_tokens = kAttnMinUnitTokensPerSlot * group_slots(num_q_heads / num_kv_heads);
    if (mfma && min_tokens < 2 * kMfmaTile)
        min_tokens = 2 * kMfmaTile;  // at least two matrix tiles per unit
    const uint64_t min_pages = (min_tokens + page_size - 1) / page_size;
    if (upages < min_pages)
        upages = min_pages;
    if (upages < 1)
        upages = 1;
    if (upages > kAttnMaxUnitPages)
        upages = kAttnMaxUnitPages;
    sh.unit_pages = (uint32_t)upages;
    sh.unit_tokens = (uint32_t)(upages * page_size);
    sh.cap_units = total_tokens / sh.unit_tokens + num_seqs;
    // The shared-prefix pass: on the matrix-core path when pages may be read
    // more than once (no streaming hint) and there are sequences to share.
    sh.shared = mfma && !stream_loads && num_seqs >= 2;
    sh.chunk_pages = (kSharedChunkTokens + page_size - 1) / page_size;
    sh.min_pages = (kMinSharedTokens + page_size - 1) / page_size;
    sh.seqs_per_block = kMfmaWaves * (G <= kMfmaRows ? kMfmaRows / G : 1);
    sh.cap_work = 0;
    if (sh.shared) {
        // shared chunks: at most ceil(L / chunk tokens) per sequence
        const uint64_t chunk_tokens = (uint64_t)sh.chunk_pages * page_size;
        sh.cap_work = total_tokens / chunk_tokens + num_seqs;
        sh.cap_units += sh.cap_work;
    }
    return sh;
}

uint64_t attention_workspace_bytes(uint64_t num_seqs, uint64_t total_tokens, uint32_t page_size,
                                   uint32_t num_kv_heads, uint32_t head_dim, uint32_t num_q_heads) {
    uint64_t need = 0;
    for (int v = 0; v < 4; ++v) {  // with and without streaming loads, 16-bit and int8 pools
        const AttentionShape sh = attention_shape(num_seqs, total_tokens, page_size, num_kv_heads,
                                                  head_dim, num_q_heads, v & 1, v & 2);
        const uint64_t n = ws_layout(num_seqs, num_q_heads, head_dim, sh).end;
        need = n > need ? n : need;
    }
    return need;
}

namespace {

// The planning kernels of a call: with the shared-prefix pass, the leading-page
// comparison and the prefix plan; above kAttnFusedSeqs sequences without it,
// the unit plan; otherwise none (the attention kernels count units
// themselves). Their results live in the workspace and depend only on the
// table, the counts and the launch shape.
hipError_t run_plan(const AttentionJob &job, const AttentionShape &sh, const WsLayout &wl,
                    hipStream_t stream) {
    unsigned char *ws = static_cast<unsigned char *>(job.workspace);
    uint32_t *unit_end = reinterpret_cast<uint32_t *>(ws + wl.unit_end);
    uint32_t *unit_seq = reinterpret_cast<uint32_t *>(ws + wl.unit_seq);
    auto at = [&](uint64_t off) { return reinterpret_cast<uint32_t *>(ws + off); };
    const bool fused = job.num_seqs <= kAttnFusedSeqs && !sh.shared;
    if (sh.shared) {
        PlanArgs pa = {};
        pa.block_table = job.block_table;
        pa.seq_ptr = job.seq_ptr;
        pa.seq_lens = job.seq_lens;
        pa.num_seqs = job.num_seqs;
        pa.page_size = job.page_size;
        pa.unit_tokens = sh.unit_tokens;
        pa.chunk_pages = sh.chunk_pages;
        pa.min_pages = sh.min_pages;
        pa.seqs_per_block = sh.seqs_per_block;
        pa.cap_units = (uint32_t)sh.cap_units;
        pa.cap_work = (uint32_t)sh.cap_work;
        pa.unit_end = unit_end;
        pa.unit_seq = unit_seq;
        pa.pre_pages = at(wl.pre_pages);
        pa.run_of = at(wl.run_of);
        pa.run_first = at(wl.run_first);
        pa.run_c = at(wl.run_c);
        pa.work_seq0 = at(wl.work_seq0);
        pa.work_chunk = at(wl.work_chunk);
        pa.nwork = at(wl.nwork);
        const uint32_t lcp_groups = (job.num_seqs + kAttnThreads / 64 - 1) / (kAttnThreads / 64);
        hipLaunchKernelGGL(job.idx64 ? attention_lcp_kernel<uint64_t>
                                     : attention_lcp_kernel<uint32_t>,
                           dim3(lcp_groups), dim3(kAttnThreads), 0, stream, pa);
        hipLaunchKernelGGL(job.idx64 ? attention_prefix_plan_kernel<uint64_t>
                                     : attention_prefix_plan_kernel<uint32_t>,
                           dim3(1), dim3(kAttnThreads), 0, stream, pa);
        return hipGetLastError();
    }
    if (!fused) {
        hipLaunchKernelGGL(job.idx64 ? attention_plan_kernel<uint64_t>
                                     : attention_plan_kernel<uint32_t>,
                           dim3(1), dim3(kAttnThreads), 0, stream, job.seq_lens, job.num_seqs,
                           sh.unit_tokens, (uint32_t)sh.cap_units, unit_end, unit_seq);
        return hipGetLastError();
    }
    return hipSuccess;
}

} // namespace

hipError_t launch_attention_plan(const AttentionJob &job, hipStream_t stream) {
    (void)hipGetLastError();  // clear errors left by earlier calls that are not ours
    const AttentionShape sh = attention_shape(job.num_seqs, job.total_tokens, job.page_size,
                                              job.num_kv_heads, job.head_dim, job.num_q_heads,
                                              job.stream_loads, job.q8);
    return run_plan(job, sh, ws_layout(job.num_seqs, job.num_q_heads, job.head_dim, sh), stream);
}

hipError_t launch_attention(const AttentionJob &job, hipStream_t stream) {
    (void)hipGetLastError();  // clear errors left by earlier calls that are not ours
    const AttentionShape sh = attention_shape(job.num_seqs, job.total_tokens, job.page_size,
                                              job.num_kv_heads, job.head_dim, job.num_q_heads,
                                              job.stream_loads, job.q8);
    const WsLayout wl = ws_layout(job.num_seqs, job.num_q_heads, job.head_dim, sh);
    unsigned char *ws = static_cast<unsigned char *>(job.workspace);
    uint32_t *unit_end = reinterpret_cast<uint32_t *>(ws + wl.unit_end);
    uint32_t *unit_seq = reinterpret_cast<uint32_t *>(ws + wl.unit_seq);
    auto at = [&](uint64_t off) { return reinterpret_cast<uint32_t *>(ws + off); };

    const bool fused = job.num_seqs <= kAttnFusedSeqs && !sh.shared;
    hipError_t e = hipSuccess;
    // planned: the workspace holds this shape's plan from launch_attention_plan
    if (!job.planned && (e = run_plan(job, sh, wl, stream)) != hipSuccess)
        return e;

    AArgs a = {};
    a.k_pool = static_cast<const unsigned char *>(job.k_pool);
    a.v_pool = static_cast<const unsigned char *>(job.v_pool);
    a.q = static_cast<const unsigned char *>(job.q);
    a.block_table = job.block_table;
    a.seq_ptr = job.seq_ptr;
    a.seq_lens = job.seq_lens;
    a.unit_end = unit_end;
    a.unit_seq = unit_seq;
    a.part_ml = reinterpret_cast<float *>(ws + wl.ml);
    a.part_acc = reinterpret_cast<float *>(ws + wl.acc);
    a.out = job.out;
    a.num_seqs = job.num_seqs;
    a.page_size = job.page_size;
    a.num_kv_heads = job.num_kv_heads;
    a.num_q_heads = job.num_q_heads;
    a.head_dim = job.head_dim;
    a.unit_tokens = sh.unit_tokens;
    a.unit_pages = sh.unit_pages;
    a.heads_per_group = sh.heads_per_group;
    a.token_lanes = sh.token_lanes;
    a.cap_units = (uint32_t)sh.cap_units;
    a.group = job.num_q_heads / job.num_kv_heads;
    a.fused = fused;
    a.qscale = job.scale * 1.4426950408889634f;  // log2(e)
    a.div_page = make_div(job.page_size);
    const uint32_t G = job.num_q_heads / job.num_kv_heads;
    a.pg_area = (uint32_t)((8 * (uint64_t)(sh.shared && sh.chunk_pages > sh.unit_pages
                                                ? sh.chunk_pages : sh.unit_pages) + 15) &
                           ~uint64_t(15));
    if (sh.shared) {
        a.shared = 1;
        a.chunk_pages = sh.chunk_pages;
        a.seqs_per_block = sh.seqs_per_block;
        a.pre_pages = at(wl.pre_pages);
        a.run_of = at(wl.run_of);
        a.work_seq0 = at(wl.work_seq0);
        a.work_chunk = at(wl.work_chunk);
        a.nwork = at(wl.nwork);
    }
    // With the shared pass the units cover the pages after each run's shared
    // part, mostly read once: streaming loads (measured 1 to 2 % faster on
    // the prefix batch); the shared items keep cached loads.
    const bool nt = job.stream_loads || sh.shared;
    a.k_scales = job.k_scales;
    a.v_scales = job.v_scales;
    e = job.q8     ? launch_attention_i<BF16, true>(a, sh, G, job.idx64, nt, stream)
        : job.bf16 ? launch_attention_i<BF16, false>(a, sh, G, job.idx64, nt, stream)
                   : launch_attention_i<F16, false>(a, sh, G, job.idx64, nt, stream);
    if (e != hipSuccess)
        return e;

    CArgs c = {};
    c.unit_end = fused ? nullptr : unit_end;
    c.seq_lens = job.seq_lens;
    c.unit_tokens = sh.unit_tokens;
    c.cap_units = (uint32_t)sh.cap_units;
    c.part_ml = a.part_ml;
    c.part_acc = a.part_acc;
    c.out = job.out;
    c.num_q_heads = job.num_q_heads;
    c.head_dim = job.head_dim;
    c.div_d = make_div(job.head_dim);
    const uint32_t per_seq = job.num_q_heads * job.head_dim / 4;  // 4 outputs per thread
    hipLaunchKernelGGL(job.idx64 ? attention_combine_kernel<uint64_t>
                                 : attention_combine_kernel<uint32_t>,
                       dim3(job.num_seqs, (per_seq + kAttnThreads - 1) / kAttnThreads),
                       dim3(kAttnThreads), 0, stream, c);
    return hipGetLastError();
}

} // namespace hp
