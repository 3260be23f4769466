// hp_kernels.hip -- gfx950 kernels for the block-paged KV layout.
//
// Source of the arithmetic: "Block-Paged Layout -- Hurray Format
// Specification", sections Element Lookup (address of token t of sequence s),
// Logical Shape (the ragged tensor is the sequences' tokens concatenated in
// order), Partial trailing page (nothing past a sequence's count is read; a
// writer should zero the unused slots), Per-page-slot parameters (one scale
// per physical page slot) and Storage Invariants (what a reader validates).
//
// Design (one GPU, HBM-bound, nothing is a contraction so no MFMA):
//  * A page of the interchange layout [N, P, H, D] is one contiguous span of
//    P*R bytes (R = H*D*elem bytes), and so is a run of consecutive tokens of
//    one sequence inside one page, on both sides of the move. The work unit
//    is such a run: `rows_per_unit` consecutive tokens (a divisor of P, so a
//    unit never crosses a page), i.e. one block-table entry and one
//    contiguous span; the host sizes it per move (8 KB and up for gather,
//    growing with the sequence count; 8 or 32 KB for scatter; 32 KB of
//    output for dequant).
//  * Work units are numbered sequence by sequence. Each workgroup owns
//    `units_per_group` consecutive units. To map a unit to its sequence it
//    needs, per sequence, the running unit count and the running token count
//    (the row where the sequence starts in the logical tensor). Up to
//    kFusedMaxSeqs sequences every workgroup rebuilds both prefix sums in LDS
//    from the token counts (a 64-lane shuffle scan per wave, wave totals
//    combined through LDS), so one launch does everything; above it, a plan
//    pass writes them to the workspace and the copy kernel reads them there.
//  * Gather, scatter and quantize-on-scatter workgroups learn their first
//    unit's sequence inside the fused scan (the owning thread publishes it
//    through LDS); dequant searches the scanned table. The block-table entry of a unit is read once
//    per unit into a scalar register; the sequence's scalars are reloaded
//    only when the walk moves to the next sequence.
//  * Copies are 16-byte vector loads and non-temporal 16-byte vector stores,
//    2, 4 or 8 loads per lane in flight (the smallest that covers a unit);
//    narrower vectors are used only when a row size or pointer forbids 16
//    bytes.
//  * Dequant reads 8 int8 values per lane and writes 8 bf16 values (16 B) per
//    lane, so both sides stay fully coalesced; the unit's per-slot scales sit
//    one per lane and are fetched with a cross-lane shuffle.
//  * Quantize-on-scatter: a wave quantizes a whole row, its extremes first
//    (combined with shuffles) and then its codes. With 16-byte vectors and
//    at most 256 sequences a workgroup is one wave and its unit one slot;
//    otherwise four waves take a unit of up to 4 slots, a row each.
#include "hp_device.h"
#include "hp_internal.h"

#include <stdint.h>

namespace hp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int B> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

#ifndef HP_COPY_UNROLL
#define HP_COPY_UNROLL 8
#endif
#ifndef HP_STORE_NT
#define HP_STORE_NT 1
#endif
constexpr int kCopyUnroll = HP_COPY_UNROLL;
constexpr int kDequantUnroll = 8;

// Loads of the moved data: non-temporal when every source byte is read once
// (a streamed pool or a scatter's source rows), cached otherwise (aliased
// pages are then fetched from HBM once and served from L2 after that).
template <bool NT, typename V>
__device__ __forceinline__ V ld_stream(const V *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
// Stores of the moved data: non-temporal by default (nothing here re-reads
// them).
template <typename V>
__device__ __forceinline__ void st_stream(V v, V *p) {
#if HP_STORE_NT
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// Device-side view of a launch. Offsets inside one unit are 32-bit (the host
// guarantees rows_per_unit * row bytes < 2^31); page and row bases are 64-bit.
struct Args {
    const void *block_table;
    const void *seq_ptr;
    const void *seq_lens;
    const void *seq_start;
    const uint32_t *g_unit_end;  // plan arrays (non-fused launches)
    const uint64_t *g_tok_begin;
    uint64_t *partials;
    uint32_t num_seqs;
    uint32_t page_size;
    uint32_t rows_per_unit;
    uint32_t units_per_page;  // page_size / rows_per_unit
    uint32_t units_per_group;
    uint32_t row_bytes;       // pool row
    uint32_t out_row_bytes;   // logical-tensor row
    uint32_t zero_tail;
    uint32_t vecs_per_row;    // dequant: input vectors per row
    Div div_vpr, div_rpc, div_page, div_upp;  // by vecs_per_row, rows_per_unit,
                                              // page_size, units_per_page
    // General dequant scheme (see CopyJob): signedness and parameters.
    uint32_t quant_unsigned;
    const float *quant_scales;
    const void *zero_points;
    uint32_t head_dim;
    uint32_t quant_channels;  // entries of a per-channel table
    Div div_hd;
    // Quantize-on-scatter: the per-slot parameters it writes.
    float *qs_scales;
    uint8_t *qs_zero_points;
    // Gated moves: the verdict words of an enqueued validation, or null.
    const unsigned long long *gate;
    uint64_t gate_tokens;
    // Pool m of the launch is moved by grid row m (blockIdx.y).
    unsigned char *pool[kMaxBatch];   // scatter writes it, gather/dequant read it
    unsigned char *rows[kMaxBatch];   // the logical tensor of pool m
    const float *scales[kMaxBatch];   // dequant: per-slot scales of pool m
};

// Units (token runs) of sequence s. Gather/dequant: ceil(L / rpc) runs
// starting at token 0. Scatter: the rpc-aligned windows of positions
// [start, start + L), extended to the end of the last page when the tail is
// zeroed.
template <Op OP>
__device__ __forceinline__ uint64_t units_of(const Args &a, uint64_t len, uint64_t start) {
    const uint64_t rpc = a.rows_per_unit;
    if (!writes_pool(OP))
        return udiv(len + rpc - 1, a.div_rpc);
    if (len == 0)
        return 0;
    const uint64_t end = start + len;
    const uint64_t w0 = udiv(start, a.div_rpc);
    const uint64_t w1 = a.zero_tail
        ? udiv(end + a.page_size - 1, a.div_page) * a.units_per_page
        : udiv(end + rpc - 1, a.div_rpc);
    return w1 - w0;
}

// Exclusive scan of (units, tokens) over the workgroup's NTH threads. Returns
// the thread's exclusive prefix; `total_*` receives the workgroup totals.
template <uint32_t NTH = kThreads>
__device__ __forceinline__ void group_exclusive_scan(uint64_t &u, uint64_t &t,
                                                     uint64_t &total_u, uint64_t &total_t) {
    __shared__ uint64_t wave_u[NTH / 64], wave_t[NTH / 64];
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t ui = u, ti = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        uint64_t un = __shfl_up(ui, d, 64);
        uint64_t tn = __shfl_up(ti, d, 64);
        if (lane >= (uint32_t)d) {
            ui += un;
            ti += tn;
        }
    }
    if (lane == 63) {
        wave_u[wave] = ui;
        wave_t[wave] = ti;
    }
    __syncthreads();
    uint64_t bu = 0, bt = 0;
    total_u = 0;
    total_t = 0;
#pragma unroll
    for (uint32_t w = 0; w < NTH / 64; ++w) {
        if (w < wave) {
            bu += wave_u[w];
            bt += wave_t[w];
        }
        total_u += wave_u[w];
        total_t += wave_t[w];
    }
    u = bu + ui - u;
    t = bt + ti - t;
    __syncthreads();  // wave_u / wave_t may be reused by the next scan
}

// Writes unit_end[s] (inclusive running unit count) and tok_begin[s]
// (exclusive running token count) for s in [s0, s1), starting from the given
// bases. Each of the NTH threads takes a contiguous run of ceil((s1-s0)/NTH)
// sequences. Ends with a barrier.
template <typename IdxT, Op OP, uint32_t NTH = kThreads, typename UE, typename TB>
__device__ __forceinline__ void scan_range(const Args &a, uint32_t s0, uint32_t s1,
                                           uint64_t ubase, uint64_t tbase, UE *unit_end,
                                           TB *tok_begin) {
    const uint32_t n = s1 - s0;
    const uint32_t per = (n + NTH - 1) / NTH;
    const uint32_t i0 = s0 + min32(n, threadIdx.x * per);
    const uint32_t i1 = s0 + min32(n, (threadIdx.x + 1) * per);
    uint64_t u = 0, t = 0;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
        const uint64_t st = (writes_pool(OP) && a.seq_start) ? ld_idx<IdxT>(a.seq_start, i) : 0;
        u += units_of<OP>(a, len, st);
        t += len;
    }
    uint64_t tu, tt;
    group_exclusive_scan<NTH>(u, t, tu, tt);
    u += ubase;
    t += tbase;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
        const uint64_t st = (writes_pool(OP) && a.seq_start) ? ld_idx<IdxT>(a.seq_start, i) : 0;
        u += units_of<OP>(a, len, st);
        unit_end[i] = (UE)u;
        tok_begin[i] = (TB)t;
        t += len;
    }
    __syncthreads();
}

// Gather and scatter workgroups find their first unit's sequence inside the
// fused scan (fused_scan_locate); dequant and quantize-on-scatter search the
// scanned table afterwards. Measured on MI355X on the decode batch: the
// in-scan lookup gains 5 % on gather and scatter (8 KB units) and loses
// 0.5 % on dequant, whose larger units make the lookup a smaller share.
// Threads per copy workgroup: quantize-on-scatter with U = 1 runs one wave
// per workgroup, one slot each (rows are then scheduled one by one instead of
// four to a workgroup); every other instance runs kThreads.
constexpr uint32_t block_threads(Op op, int u) {
    return (op == Op::ScatterQuant && u == 1) ? 64u : kThreads;
}

constexpr bool locate_in_scan(Op op) {
    return op == Op::Gather || op == Op::Scatter || op == Op::ScatterQuant;
}

// What a workgroup needs about the sequence that holds its first unit.
struct FirstSeq {
    uint64_t len, sp, start, tb;
    uint32_t s, ubeg, uend, pad;
};

// Sequences per thread whose count, start and seq_ptr stay in registers
// between the two passes of the fused scan (up to threads * this many
// sequences; beyond, the second pass reads them again).
constexpr uint32_t kScanRegs = 4;

// The fused scan of a copy workgroup: writes unit_end[s] and tok_begin[s] for
// every sequence, like scan_range, and the thread whose sequence holds unit
// g0 also writes that sequence's values to `first`. The workgroup then starts
// moving after one pass of loads (counts and seq_ptr together) and two
// barriers, with no search and no further load. Ends with a barrier.
template <typename IdxT, Op OP, uint32_t NTH = kThreads>
__device__ __forceinline__ void fused_scan_locate(const Args &a, uint32_t S, uint32_t g0,
                                                  uint32_t *unit_end, uint64_t *tok_begin,
                                                  FirstSeq *first) {
    const uint32_t per = (S + NTH - 1) / NTH;  // wave-uniform
    const uint32_t i0 = min32(S, threadIdx.x * per);
    const uint32_t i1 = min32(S, (threadIdx.x + 1) * per);
    const bool with_start = writes_pool(OP) && a.seq_start;
    uint64_t u = 0, t = 0;
    uint64_t lenr[kScanRegs], str[kScanRegs], spr[kScanRegs];
    if (per <= kScanRegs) {
        // Loads of every held sequence at once (an index past S re-reads the
        // last entry; its values are not used).
#pragma unroll
        for (uint32_t k = 0; k < kScanRegs; ++k) {
            if (k < per) {
                const uint32_t i = min32(i0 + k, S - 1);
                lenr[k] = ld_idx<IdxT>(a.seq_lens, i);
                str[k] = with_start ? ld_idx<IdxT>(a.seq_start, i) : 0;
                spr[k] = ld_idx<IdxT>(a.seq_ptr, i);
            }
        }
#pragma unroll
        for (uint32_t k = 0; k < kScanRegs; ++k) {
            if (i0 + k < i1) {
                u += units_of<OP>(a, lenr[k], str[k]);
                t += lenr[k];
            }
        }
    } else {
        for (uint32_t i = i0; i < i1; ++i) {
            const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
            u += units_of<OP>(a, len, with_start ? ld_idx<IdxT>(a.seq_start, i) : 0);
            t += len;
        }
    }
    uint64_t tu, tt;
    group_exclusive_scan<NTH>(u, t, tu, tt);
    if (per <= kScanRegs) {
#pragma unroll
        for (uint32_t k = 0; k < kScanRegs; ++k) {
            const uint32_t i = i0 + k;
            if (i < i1) {
                const uint64_t ub = u;
                u += units_of<OP>(a, lenr[k], str[k]);
                unit_end[i] = (uint32_t)u;
                tok_begin[i] = t;
                if (g0 >= ub && g0 < u)
                    *first = FirstSeq{lenr[k], spr[k], str[k], t, i, (uint32_t)ub, (uint32_t)u, 0};
                t += lenr[k];
            }
        }
    } else {
        for (uint32_t i = i0; i < i1; ++i) {
            const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
            const uint64_t st = with_start ? ld_idx<IdxT>(a.seq_start, i) : 0;
            const uint64_t ub = u;
            u += units_of<OP>(a, len, st);
            unit_end[i] = (uint32_t)u;
            tok_begin[i] = t;
            if (g0 >= ub && g0 < u)
                *first = FirstSeq{len, ld_idx<IdxT>(a.seq_ptr, i), st, t, i, (uint32_t)ub,
                                  (uint32_t)u, 0};
            t += len;
        }
    }
    __syncthreads();
}

// ---- span movers -------------------------------------------------------------

// U loads per lane in flight, then the U stores; U * kThreads vectors per
// round.
template <int U, int VEC, bool NTL>
__device__ __forceinline__ void copy_rounds(const typename Vec<VEC>::T *__restrict__ s,
                                            typename Vec<VEC>::T *__restrict__ d, uint32_t n) {
    using V = typename Vec<VEC>::T;
    for (uint32_t base = threadIdx.x; base < n; base += kThreads * U) {
        V tmp[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint32_t i = base + j * kThreads;
            if (i < n)
                tmp[j] = ld_stream<NTL>(s + i);
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const uint32_t i = base + j * kThreads;
            if (i < n)
                st_stream(tmp[j], d + i);
        }
    }
}

// U loads in flight per lane. The launch picks the smallest U of 2, 4, 8
// that covers one work unit: loads past a unit's end sat behind branches
// that still cost issue slots and waits (decode batch, 8 KB units: U = 2 is
// 5 % ahead of U = 8 on gather and scatter, and a run-time choice between the
// two bodies inside one kernel lost that again).
template <int U, int VEC, bool NTL>
__device__ __forceinline__ void copy_span(const unsigned char *__restrict__ src,
                                          unsigned char *__restrict__ dst, uint32_t nbytes) {
    using V = typename Vec<VEC>::T;
    copy_rounds<U, VEC, NTL>(reinterpret_cast<const V *>(src), reinterpret_cast<V *>(dst),
                             nbytes / VEC);
}

template <int VEC>
__device__ __forceinline__ void zero_span(unsigned char *__restrict__ dst, uint32_t nbytes) {
    using V = typename Vec<VEC>::T;
    V *d = reinterpret_cast<V *>(dst);
    const uint32_t n = nbytes / VEC;
    const V z = V(0);
    for (uint32_t i = threadIdx.x; i < n; i += kThreads)
        st_stream(z, d + i);
}

// Dequantises `rows` rows of R_in int8 values into bf16. `scale_row` points at
// the scale of the unit's first slot; rows <= 64, so lane r holds row r's
// scale and every lane fetches its row's scale from that lane.
template <int VIN>
__device__ __forceinline__ void dequant_span(const Args &a, const unsigned char *__restrict__ src,
                                             const float *__restrict__ scale_row,
                                             unsigned char *__restrict__ dst, uint32_t rows) {
    using VI = typename Vec<VIN>::T;
    const uint32_t lane = threadIdx.x & 63;
    const float my_scale = lane < rows ? scale_row[lane] : 0.0f;
    const uint32_t n = rows * a.vecs_per_row;
    const VI *s = reinterpret_cast<const VI *>(src);
    // The trip count is the same for every lane: the shuffle below reads the
    // scale from another lane, which must still be active.
    for (uint32_t b0 = 0; b0 < n; b0 += kThreads * kDequantUnroll) {
        const uint32_t base = b0 + threadIdx.x;
        VI q[kDequantUnroll];
#pragma unroll
        for (int j = 0; j < kDequantUnroll; ++j) {
            const uint32_t i = base + j * kThreads;
            if (i < n)
                q[j] = ld_stream<false>(s + i);
        }
#pragma unroll
        for (int j = 0; j < kDequantUnroll; ++j) {
            const uint32_t i = base + j * kThreads;
            const uint32_t row = udiv32(i, a.div_vpr);
            const float sc = __shfl(my_scale, (int)row, 64);
            if (i < n) {
                if constexpr (VIN == 8) {
                    const u32x2 w = q[j];
                    u32x4 o;
                    o.x = pack_bf16x2(sbyte(w.x, 0) * sc, sbyte(w.x, 1) * sc);
                    o.y = pack_bf16x2(sbyte(w.x, 2) * sc, sbyte(w.x, 3) * sc);
                    o.z = pack_bf16x2(sbyte(w.y, 0) * sc, sbyte(w.y, 1) * sc);
                    o.w = pack_bf16x2(sbyte(w.y, 2) * sc, sbyte(w.y, 3) * sc);
                    st_stream(o, reinterpret_cast<u32x4 *>(dst) + i);
                } else if constexpr (VIN == 4) {
                    const uint32_t w = q[j];
                    u32x2 o;
                    o.x = pack_bf16x2(sbyte(w, 0) * sc, sbyte(w, 1) * sc);
                    o.y = pack_bf16x2(sbyte(w, 2) * sc, sbyte(w, 3) * sc);
                    st_stream(o, reinterpret_cast<u32x2 *>(dst) + i);
                } else if constexpr (VIN == 2) {
                    const uint32_t w = q[j];
                    const uint32_t o = pack_bf16x2(sbyte(w, 0) * sc, sbyte(w, 1) * sc);
                    st_stream(o, reinterpret_cast<uint32_t *>(dst) + i);
                } else {
                    const uint16_t o = to_bf16(sbyte(q[j], 0) * sc);
                    st_stream(o, reinterpret_cast<uint16_t *>(dst) + i);
                }
            }
        }
    }
}

// Order in which workgroups take work. The dispatcher hands consecutive
// workgroup IDs to the 8 XCDs in turn; with the remap, the workgroups that
// land on one XCD take one contiguous range of work units (a bijection on
// [0, groups)), so neighbouring units of one page share that XCD's L2.
// Measured on MI355X (decode batch, same-box A/B): the streamed scatter gains
// 4 % and quantize-on-scatter 1-3 % (both write random pages); the gather
// loses 0.7 % and the small cached scatter of an append 2x, so only those two
// take it.
template <bool REMAP>
__device__ __forceinline__ uint32_t group_order(uint32_t b, uint32_t groups) {
    if constexpr (REMAP) {
        constexpr uint32_t kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each
        const uint32_t per = (groups + kXcds - 1) / kXcds;  // groups on the fullest XCDs
        const uint32_t full = groups - (per - 1) * kXcds;   // XCDs that get `per` groups
        const uint32_t xcd = b % kXcds, local = b / kXcds;
        return xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
    } else {
        (void)groups;
        return b;
    }
}

// ---- dequant under any accepted scheme ----------------------------------------
//
// [Hurray] Per-scheme composition: out = bf16(fp32(q - zp) * scale). q - zp
// is an integer of at most 9 bits, so the float difference below is exact and
// the product rounds once, as the definition asks. A uint8 pool takes the
// signed path with the top bit of both q and zp flipped: (q - 128) - (zp - 128)
// is the same difference. Without zero points zp is 0 (-128 after the flip).
// QM: 0 per-slot, 1 per-tensor, 2 per-head, 3 per-head_dim parameters.

// Zero point k as a float, with the flip applied.
__device__ __forceinline__ float zp_at(const Args &a, uint64_t k, uint32_t flip) {
    const uint32_t b = a.zero_points ? static_cast<const uint8_t *>(a.zero_points)[k] : 0u;
    return sbyte(b ^ flip, 0);
}

// The VIN bytes of an input vector as 32-bit words (low bytes first).
template <int VIN>
__device__ __forceinline__ void to_words(const typename Vec<VIN>::T &v, uint32_t (&w)[(VIN + 3) / 4]) {
    if constexpr (VIN == 8) {
        w[0] = v.x;
        w[1] = v.y;
    } else {
        w[0] = (uint32_t)v;
    }
}

// VIN consecutive scales starting at p (p aligned to 4 * VIN bytes). The
// vector is copied whole: clang's __builtin_bit_cast of an ext-vector element
// (v.y) reads element 0, so elements are never bit-cast one by one.
template <int VIN>
__device__ __forceinline__ void load_scales(const float *__restrict__ p, float (&o)[VIN]) {
    if constexpr (VIN >= 4) {
#pragma unroll
        for (int c = 0; c < VIN / 4; ++c) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(p)[c];
            __builtin_memcpy(&o[4 * c], &v, sizeof v);
        }
    } else if constexpr (VIN == 2) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
        __builtin_memcpy(&o[0], &v, sizeof v);
    } else {
        o[0] = p[0];
    }
}

// One channel's scale and zero point (flipped, as a float): the per-channel
// tables are staged in LDS in this form when they have at most
// kQuantLdsMax entries.
struct QParam {
    float scale, zp;
};
constexpr uint32_t kQuantLdsMax = 2048;

// QM 2 and 3 read the staged table; QM 4 and 5 are the same schemes (per-head,
// per-head_dim) with the parameters read from global memory.
constexpr int channel_axis(int qm) { return qm == 4 ? 2 : qm == 5 ? 3 : qm; }

// VIN consecutive table entries (LDS, 16-byte aligned when VIN >= 2).
template <int VIN>
__device__ __forceinline__ void lds_params(const QParam *t, float (&sc)[VIN], float (&zf)[VIN]) {
    QParam e[VIN];
    if constexpr (VIN >= 2) {
#pragma unroll
        for (int c = 0; c < VIN / 2; ++c) {
            const u32x4 v = reinterpret_cast<const u32x4 *>(t)[c];
            __builtin_memcpy(&e[2 * c], &v, sizeof v);
        }
    } else {
        e[0] = t[0];
    }
#pragma unroll
    for (int k = 0; k < VIN; ++k) {
        sc[k] = e[k].scale;
        zf[k] = e[k].zp;
    }
}

// Scales and (flipped) zero points of the VIN elements that start at element
// e0 of a row, for the per-channel schemes. When head_dim is a multiple of
// VIN the vector lies inside one head: one parameter (per-head) or VIN
// consecutive ones (per-head_dim); otherwise each element finds its own.
template <int VIN, int QM>
__device__ __forceinline__ void channel_params(const Args &a, const QParam *tab, uint32_t e0,
                                               uint32_t flip, float (&sc)[VIN], float (&zf)[VIN]) {
    constexpr int AX = channel_axis(QM);
    constexpr bool IN_LDS = QM == 2 || QM == 3;
    const uint32_t D = a.head_dim;
    auto one = [&](uint32_t c, float &sv, float &zv) {
        if constexpr (IN_LDS) {
            const QParam p = tab[c];
            sv = p.scale;
            zv = p.zp;
        } else {
            sv = a.quant_scales[c];
            zv = zp_at(a, c, flip);
        }
    };
    if ((D & (VIN - 1)) == 0) {
        const uint32_t h = udiv32(e0, a.div_hd);
        if constexpr (AX == 2) {
            float sv, zv;
            one(h, sv, zv);
#pragma unroll
            for (int k = 0; k < VIN; ++k) {
                sc[k] = sv;
                zf[k] = zv;
            }
        } else if constexpr (IN_LDS) {
            lds_params<VIN>(tab + (e0 - h * D), sc, zf);
        } else {
            const uint32_t d0 = e0 - h * D;
            load_scales<VIN>(a.quant_scales + d0, sc);
            uint32_t zw[(VIN + 3) / 4] = {};
            if (a.zero_points)
                to_words<VIN>(*reinterpret_cast<const typename Vec<VIN>::T *>(
                                  static_cast<const uint8_t *>(a.zero_points) + d0),
                              zw);
#pragma unroll
            for (int k = 0; k < VIN; ++k)
                zf[k] = sbyte(zw[k / 4] ^ (flip * 0x01010101u), k % 4);
        }
    } else {
#pragma unroll
        for (int k = 0; k < VIN; ++k) {
            const uint32_t e = e0 + k;
            const uint32_t h = udiv32(e, a.div_hd);
            one(AX == 2 ? h : e - h * D, sc[k], zf[k]);
        }
    }
}

// One tile of kDequantUnroll vectors per thread starting at vector `base`.
// FULL: every vector of the tile is in range, so loads and stores need no
// guard and the compiler keeps all loads in flight at once; the tail tile
// (FULL = false) checks each index.
template <int VIN, int QM, bool FULL>
__device__ __forceinline__ void dequant_tile(const Args &a, const typename Vec<VIN>::T *__restrict__ s,
                                             unsigned char *__restrict__ dst, uint32_t base,
                                             uint32_t n, float my_scale, float my_zp, float t_scale,
                                             float t_zp, uint32_t flip, const QParam *tab) {
    using VI = typename Vec<VIN>::T;
    using VO = typename Vec<2 * VIN>::T;  // VIN bf16 values
    VI q[kDequantUnroll];
#pragma unroll
    for (int j = 0; j < kDequantUnroll; ++j) {
        const uint32_t i = base + j * kThreads;
        if (FULL || i < n)
            q[j] = ld_stream<false>(s + i);
    }
    const uint32_t fw = flip * 0x01010101u;
#pragma unroll
    for (int j = 0; j < kDequantUnroll; ++j) {
        const uint32_t i = base + j * kThreads;
        const uint32_t row = udiv32(i, a.div_vpr);
        float rs = 0.0f, rz = 0.0f;
        if constexpr (QM == 0) {  // every lane takes part in the shuffles
            rs = __shfl(my_scale, (int)row, 64);
            rz = __shfl(my_zp, (int)row, 64);
        }
        if (!FULL && i >= n)
            continue;
        float sc[VIN], zf[VIN];
        if constexpr (QM == 0 || QM == 1) {
#pragma unroll
            for (int k = 0; k < VIN; ++k) {
                sc[k] = QM == 0 ? rs : t_scale;
                zf[k] = QM == 0 ? rz : t_zp;
            }
        } else {
            channel_params<VIN, QM>(a, tab, (i - row * a.vecs_per_row) * VIN, flip, sc, zf);
        }
        uint32_t w[(VIN + 3) / 4];
        to_words<VIN>(q[j], w);
        if constexpr (VIN == 1) {
            st_stream(to_bf16((sbyte(w[0] ^ fw, 0) - zf[0]) * sc[0]),
                      reinterpret_cast<uint16_t *>(dst) + i);
        } else {
            uint32_t o[VIN / 2];
#pragma unroll
            for (int k = 0; k < VIN; k += 2)
                o[k / 2] = pack_bf16x2((sbyte(w[k / 4] ^ fw, k % 4) - zf[k]) * sc[k],
                                       (sbyte(w[k / 4] ^ fw, k % 4 + 1) - zf[k + 1]) * sc[k + 1]);
            VO packed;
            __builtin_memcpy(&packed, o, sizeof packed);
            st_stream(packed, reinterpret_cast<VO *>(dst) + i);
        }
    }
}

// Dequantises `rows` rows (rows <= 64) of a unit. Per-slot parameters are held
// one per lane and fetched by shuffle. `slot0` is the global slot index
// (phys * page_size + slot) of the unit's first row and `slot_scales` its
// scale (per-slot scheme only); `tab` is the staged channel table (QM 2, 3).
template <int VIN, int QM>
__device__ __forceinline__ void dequant_span_q(const Args &a, const unsigned char *__restrict__ src,
                                               const float *__restrict__ slot_scales,
                                               uint64_t slot0, unsigned char *__restrict__ dst,
                                               uint32_t rows, const QParam *tab) {
    using VI = typename Vec<VIN>::T;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t flip = a.quant_unsigned ? 0x80u : 0u;
    float my_scale = 0.0f, my_zp = 0.0f, t_scale = 0.0f, t_zp = 0.0f;
    if constexpr (QM == 0) {
        if (lane < rows) {
            my_scale = slot_scales[lane];
            my_zp = zp_at(a, slot0 + lane, flip);
        }
    } else if constexpr (QM == 1) {
        t_scale = a.quant_scales[0];
        t_zp = zp_at(a, 0, flip);
    }
    const uint32_t n = rows * a.vecs_per_row;
    const VI *s = reinterpret_cast<const VI *>(src);
    constexpr uint32_t kTile = kThreads * kDequantUnroll;
    uint32_t b0 = 0;
    for (; b0 + kTile <= n; b0 += kTile)
        dequant_tile<VIN, QM, true>(a, s, dst, b0 + threadIdx.x, n, my_scale, my_zp, t_scale, t_zp,
                                    flip, tab);
    if (b0 < n)
        dequant_tile<VIN, QM, false>(a, s, dst, b0 + threadIdx.x, n, my_scale, my_zp, t_scale, t_zp,
                                     flip, tab);
}

// ---- quantize-on-scatter --------------------------------------------------------
//
// One written slot's row (n = row_bytes values, source element type SRC:
// 0 f16, 1 bf16, 2 f32) quantized by the whole workgroup ([Hurray] Per-page-
// slot parameters: the scale, and for an asymmetric scheme the zero point,
// of physical slot phys * page_size + slot). Reading of the formulas, every
// step one binary32 operation rounded to nearest even:
//   symmetric int8:   scale = amax / 127, q = clamp(rint(x / scale), -127, 127)
//   asymmetric uint8: lo = min(0, x), hi = max(0, x), scale = (hi - lo) / 255,
//                     z = clamp(rint(-lo / scale), 0, 255),
//                     q = clamp(rint(x / scale) + z, 0, 255)
// and a zero scale gives zero codes (and zero point). Division is the IEEE
// division (__fdiv_rn), rint rounds half to even.

constexpr int kQuantKeep = 8;  // vectors per lane held in registers between the passes

// Raw bits of one vector of a source row (8 values: 16 bytes of f16/bf16 or
// 32 of f32), or of a single value. A row's kept vectors are held in this
// form and unpacked to binary32 where they are used: 4 registers per vector
// of 16-bit values instead of 8.
template <int SRC, int VE>
struct QVec {
    u32x4 w[(VE == 8 && SRC == 2) ? 2 : 1];
};
template <int SRC, int VE>
__device__ __forceinline__ QVec<SRC, VE> load_qvec(const unsigned char *row, uint32_t i) {
    QVec<SRC, VE> v;
    if constexpr (VE == 1) {
        v.w[0] = u32x4(0);
        v.w[0].x = SRC == 2 ? reinterpret_cast<const uint32_t *>(row)[i]
                            : (uint32_t)reinterpret_cast<const uint16_t *>(row)[i];
    } else if constexpr (SRC == 2) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(row) + 2 * i;
        v.w[0] = ld_stream<true>(p);
        v.w[1] = ld_stream<true>(p + 1);
    } else {
        v.w[0] = ld_stream<true>(reinterpret_cast<const u32x4 *>(row) + i);
    }
    return v;
}
template <int SRC, int VE>
__device__ __forceinline__ void unpack_qvec(const QVec<SRC, VE> &v, float (&f)[VE]) {
    if constexpr (VE == 1) {
        const uint32_t h = v.w[0].x;
        f[0] = SRC == 2 ? __builtin_bit_cast(float, h)
             : SRC == 1 ? __builtin_bit_cast(float, h << 16)
                        : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    } else if constexpr (SRC == 2) {
        __builtin_memcpy(&f[0], &v.w[0], 16);
        __builtin_memcpy(&f[4], &v.w[1], 16);
    } else {
        uint32_t w[4];
        __builtin_memcpy(w, &v.w[0], 16);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (SRC == 1) {
                f[2 * k] = __builtin_bit_cast(float, w[k] << 16);
                f[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
            } else {
                f[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] & 0xffffu));
                f[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[k] >> 16));
            }
        }
    }
}
template <int SRC, int VE>
__device__ __forceinline__ void load_row_vec(const unsigned char *row, uint32_t i, float (&f)[VE]) {
    unpack_qvec<SRC, VE>(load_qvec<SRC, VE>(row, i), f);
}

// Quotients x / s rounded to nearest even, as one IEEE binary32 division
// would give them. FAST: y is RN(1/s); the first remainder step makes the
// product x * y a faithful quotient, and by Markstein's theorem (correctly
// rounded reciprocal, faithful quotient, exact FMA remainder) the second
// step rounds it correctly. This holds for s in [2^-100, 2^100] and for
// quotients of magnitude at least 1/4 (smaller ones round to code 0 on
// either path); s == 0 with y == 0 gives 0 for every finite x. Any other
// scale takes the division itself.
template <bool FAST>
__device__ __forceinline__ float quotient(float x, float s, float y) {
#pragma clang fp contract(off)
    if constexpr (FAST) {
        const float q0 = x * y;
        const float q1 = __builtin_fmaf(__builtin_fmaf(-s, q0, x), y, q0);
        return __builtin_fmaf(__builtin_fmaf(-s, q1, x), y, q1);
    } else {
        return __fdiv_rn(x, s);
    }
}

// The code of one value in the low byte of the result: the quotient's
// nearest integer (ties to even), plus the zero point, clamped. Adding
// 1.5 * 2^23 to a binary32 value of magnitude below 2^22 rounds it to an
// integer, ties to even (the sum's ulp is 1 and 1.5 * 2^23 is even), and
// leaves that integer in the sum's low bits; quotients here stay below 2^9
// in magnitude (|x| is at most about 255 scales). Symmetric codes are
// clamped first, which gives the same integer since the bounds are integers.
// zb is the bit pattern of 1.5 * 2^23 minus the zero point.
template <bool ASYM, bool FAST>
__device__ __forceinline__ uint32_t code_bits(float x, float s, float y, int32_t zb) {
#pragma clang fp contract(off)
    constexpr float kRound = 0x1.8p23f;
    const float q = quotient<FAST>(x, s, y);
    if constexpr (ASYM) {
        const int32_t c = (int32_t)__builtin_bit_cast(uint32_t, q + kRound) - zb;
        return (uint32_t)(c < 0 ? 0 : (c > 255 ? 255 : c));
    } else {
        const float t = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
        return __builtin_bit_cast(uint32_t, t + kRound);  // low byte: two's complement
    }
}

// Low bytes of a, b, c, d as one word (a in byte 0).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c,
                                                   uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

template <bool ASYM, int VE, bool FAST>
__device__ __forceinline__ void store_codes(unsigned char *dst, uint32_t i, const float (&f)[VE],
                                            float s, float y, int32_t zb) {
    uint32_t c[VE];
#pragma unroll
    for (int k = 0; k < VE; ++k)
        c[k] = code_bits<ASYM, FAST>(f[k], s, y, zb);
    if constexpr (VE == 8) {
        u32x2 v;
        v.x = pack_low_bytes(c[0], c[1], c[2], c[3]);
        v.y = pack_low_bytes(c[4], c[5], c[6], c[7]);
        st_stream(v, reinterpret_cast<u32x2 *>(dst) + i);
    } else {
        st_stream((unsigned char)c[0], dst + i);
    }
}

template <bool ASYM, int VE>
__device__ __forceinline__ void fold_extremes(const float (&f)[VE], float &lo, float &hi) {
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        if constexpr (ASYM) {
            lo = __builtin_fminf(lo, f[e]);
            hi = __builtin_fmaxf(hi, f[e]);
        } else {
            hi = __builtin_fmaxf(hi, __builtin_fabsf(f[e]));
        }
    }
}

constexpr int kQuantReread = 4;  // vectors per lane in flight when a row is read again

// Writes the codes of a row whose extremes are known: the kept vectors
// first, then the rest of the row, read again kQuantReread vectors per lane
// at a time. An index past the row is clamped to the row's last vector for
// the load and for the store alike: that lane writes the same codes to the
// same bytes as the lane that owns them, so no access is predicated and the
// stores of a lane need not wait for each other.
template <int SRC, bool ASYM, int VE, bool FAST>
__device__ __forceinline__ void emit_row(const unsigned char *__restrict__ src,
                                         unsigned char *__restrict__ dst, uint32_t nv,
                                         uint32_t lane, const QVec<SRC, VE> (&keep)[kQuantKeep],
                                         float s, float y, int32_t zb) {
#pragma unroll
    for (int k = 0; k < kQuantKeep; ++k) {
        // unpack again: an empty asm hides that the first pass already did,
        // so the compiler keeps the raw words rather than 8 binary32 values
        QVec<SRC, VE> v = keep[k];
#pragma unroll
        for (int j = 0; j < (int)(sizeof(v.w) / sizeof(v.w[0])); ++j)
            asm volatile("" : "+v"(v.w[j]));
        float f[VE];
        unpack_qvec<SRC, VE>(v, f);
        store_codes<ASYM, VE, FAST>(dst, min32(lane + k * 64, nv - 1), f, s, y, zb);
    }
    for (uint32_t b = kQuantKeep * 64; b < nv; b += kQuantReread * 64) {
        float f[kQuantReread][VE];
#pragma unroll
        for (int k = 0; k < kQuantReread; ++k)
            load_row_vec<SRC, VE>(src, min32(b + lane + k * 64, nv - 1), f[k]);
#pragma unroll
        for (int k = 0; k < kQuantReread; ++k)
            store_codes<ASYM, VE, FAST>(dst, min32(b + lane + k * 64, nv - 1), f[k], s, y, zb);
    }
}

// One row per wave: the row's values are spread over the wave's 64 lanes, the
// first kQuantKeep vectors of each lane stay in registers between the two
// passes (the rest are read again), and the row's extremes are combined
// with shuffles alone. Loads are never predicated, so each lane's loads are
// all in flight together.
template <int VEC, int QM>
__device__ __forceinline__ void quant_row(const Args &a, const unsigned char *__restrict__ src,
                                          unsigned char *__restrict__ dst, uint64_t slot) {
#pragma clang fp contract(off)
    constexpr int SRC = QM >> 1;
    constexpr bool ASYM = QM & 1;
    constexpr int VE = VEC == 16 ? 8 : 1;  // values per vector
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t nv = a.row_bytes / VE;  // at least 1
    QVec<SRC, VE> keep[kQuantKeep];
    float lo = 0.0f, hi = 0.0f;  // symmetric: hi is the largest |x|
    // a clamped index repeats the row's last vector: it cannot move an extreme
#pragma unroll
    for (int k = 0; k < kQuantKeep; ++k)
        keep[k] = load_qvec<SRC, VE>(src, min32(lane + k * 64, nv - 1));
#pragma unroll
    for (int k = 0; k < kQuantKeep; ++k) {
        float f[VE];
        unpack_qvec<SRC, VE>(keep[k], f);
        fold_extremes<ASYM, VE>(f, lo, hi);
    }
    for (uint32_t b = kQuantKeep * 64; b < nv; b += kQuantReread * 64) {
        float f[kQuantReread][VE];
#pragma unroll
        for (int k = 0; k < kQuantReread; ++k)
            load_row_vec<SRC, VE>(src, min32(b + lane + k * 64, nv - 1), f[k]);
#pragma unroll
        for (int k = 0; k < kQuantReread; ++k)
            fold_extremes<ASYM, VE>(f[k], lo, hi);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        if constexpr (ASYM)
            lo = __builtin_fminf(lo, __shfl_xor(lo, o, 64));
        hi = __builtin_fmaxf(hi, __shfl_xor(hi, o, 64));
    }
    // every lane holds the same extremes: make them wave-uniform
    lo = __builtin_bit_cast(float, uni(__builtin_bit_cast(uint32_t, lo)));
    hi = __builtin_bit_cast(float, uni(__builtin_bit_cast(uint32_t, hi)));
    const float sc = ASYM ? __fdiv_rn(hi - lo, 255.0f) : __fdiv_rn(hi, 127.0f);
    const float z = (ASYM && sc != 0.0f)
                        ? __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fdiv_rn(-lo, sc)), 0.0f),
                                          255.0f)
                        : 0.0f;
    const int32_t zb = (int32_t)__builtin_bit_cast(uint32_t, 0x1.8p23f) - (int32_t)z;
    if (sc == 0.0f || (sc >= 0x1p-100f && sc <= 0x1p100f)) {
        const float y = sc == 0.0f ? 0.0f : __fdiv_rn(1.0f, sc);
        emit_row<SRC, ASYM, VE, true>(src, dst, nv, lane, keep, sc, y, zb);
    } else {
        // scales this small or large are rare: read the row again, one
        // vector at a time, and divide
#pragma unroll 1
        for (uint32_t i = lane; i < nv; i += 64) {
            float f[VE];
            load_row_vec<SRC, VE>(src, i, f);
            store_codes<ASYM, VE, false>(dst, i, f, sc, 0.0f, zb);
        }
    }
    if (lane == 0) {
        a.qs_scales[slot] = sc;
        if constexpr (ASYM)
            a.qs_zero_points[slot] = (uint8_t)(int32_t)z;
    }
}

// Bytes of the fused path's LDS sequence table (8 + 4 bytes per sequence),
// rounded up so that what follows it is 16-byte aligned.
__host__ __device__ constexpr size_t lds_table_bytes(uint32_t S) {
    return (12 * (size_t)S + 15) & ~size_t(15);
}

// ---- the copy kernel -----------------------------------------------------------

// One kernel for all three moves. FUSED: per-sequence offsets rebuilt in LDS
// (dynamic LDS = 8*S + 4*S bytes); otherwise read from the plan arrays.
template <typename IdxT, Op OP, int VEC, bool FUSED, bool NTL, int QM = -1, int U = kCopyUnroll>
__global__ __launch_bounds__(block_threads(OP, U)) void copy_kernel(Args a) {
    constexpr uint32_t NTH = block_threads(OP, U);
    extern __shared__ __align__(16) unsigned char lds[];
    const uint32_t S = a.num_seqs;
    const uint32_t *unit_end;
    const uint64_t *tok_begin;
    // Per-channel dequant parameters, staged once per workgroup after the
    // sequence table (QM 2, 3).
    const QParam *tab = nullptr;
    if constexpr (OP == Op::Dequant && (QM == 2 || QM == 3)) {
        QParam *t = reinterpret_cast<QParam *>(lds + (FUSED ? lds_table_bytes(S) : 0));
        const uint32_t flip = a.quant_unsigned ? 0x80u : 0u;
        for (uint32_t c = threadIdx.x; c < a.quant_channels; c += NTH)
            t[c] = QParam{a.quant_scales[c], zp_at(a, c, flip)};
        __syncthreads();
        tab = t;
    }
    // A gated launch reads the verdict of the validation enqueued before it
    // ([Hurray] Storage Invariants: a violating descriptor is rejected). The
    // words are loaded here, beside the scan's loads, and tested before the
    // first unit: a rejected launch reads no block-table entry, pool row or
    // logical row and writes nothing.
    uint64_t gate_key = ~0ull, gate_sum = a.gate_tokens;
    if (a.gate) {
        gate_key = a.gate[0];
        gate_sum = a.gate[1];
    }
    const uint32_t g0 =
        group_order<(OP == Op::Scatter && NTL) || OP == Op::ScatterQuant>(blockIdx.x, gridDim.x) *
        a.units_per_group;
    __shared__ FirstSeq first;
    if constexpr (FUSED) {
        uint64_t *tb = reinterpret_cast<uint64_t *>(lds);
        uint32_t *ue = reinterpret_cast<uint32_t *>(lds + 8 * (size_t)S);
        if constexpr (locate_in_scan(OP))
            fused_scan_locate<IdxT, OP, NTH>(a, S, g0, ue, tb, &first);
        else
            scan_range<IdxT, OP, NTH>(a, 0, S, 0, 0, ue, tb);
        unit_end = ue;
        tok_begin = tb;
    } else {
        unit_end = a.g_unit_end;
        tok_begin = a.g_tok_begin;
    }
    const uint32_t total = uni(unit_end[S - 1]);
    if (g0 >= total)
        return;
    if (uni64(gate_key) != ~0ull || uni64(gate_sum) != a.gate_tokens)
        return;
    const uint32_t g1 = min32(g0 + a.units_per_group, total);

    const uint32_t P = a.page_size, rpc = a.rows_per_unit;
    unsigned char *const pool = a.pool[blockIdx.y];
    unsigned char *const rowsp = a.rows[blockIdx.y];
    uint32_t s = 0, ubeg = 0, uend = 0;
    uint64_t len = 0, sp = 0, start = 0, tb = 0;
    auto load_seq = [&](uint32_t q) {
        ubeg = q ? uni(unit_end[q - 1]) : 0;
        uend = uni(unit_end[q]);
        tb = uni64(tok_begin[q]);
        len = uni64(ld_idx<IdxT>(a.seq_lens, q));
        sp = uni64(ld_idx<IdxT>(a.seq_ptr, q));
        start = (writes_pool(OP) && a.seq_start) ? uni64(ld_idx<IdxT>(a.seq_start, q)) : 0;
    };
    if (FUSED && locate_in_scan(OP)) {
        // Written by the thread whose sequence holds unit g0 (g0 < total, so
        // there is one).
        s = uni(first.s);
        ubeg = uni(first.ubeg);
        uend = uni(first.uend);
        tb = uni64(first.tb);
        len = uni64(first.len);
        sp = uni64(first.sp);
        start = uni64(first.start);
    } else {
        // First sequence whose units reach past g0.
        uint32_t lo = 0, hi = S - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) >> 1;
            if (unit_end[mid] > g0)
                hi = mid;
            else
                lo = mid + 1;
        }
        s = uni(lo);
        load_seq(s);
    }

    for (uint32_t g = g0; g < g1; ++g) {
        while (g >= uend) {
            ++s;
            load_seq(s);
        }
        const uint32_t u = g - ubeg;
        if constexpr (OP == Op::ScatterQuant) {
            // Window w of rows_per_unit positions of one page: wave k takes
            // positions w * rpc + k, + k + waves, ... and quantizes each new
            // token there, or clears it when it is a tail slot.
            const uint64_t w = udiv(start, a.div_rpc) + u;
            const uint64_t q = udiv(w, a.div_upp);
            const uint64_t phys = uni64(ld_idx<IdxT>(a.block_table, sp + q));
            const uint64_t end = start + len;
            const uint64_t zend = a.zero_tail ? udiv(end + P - 1, a.div_page) * P : end;
            const uint32_t lane = threadIdx.x & 63;
            for (uint32_t r = threadIdx.x >> 6; r < rpc; r += NTH / 64) {
                const uint64_t pos = w * rpc + r;
                const uint64_t slot = phys * P + (pos - q * P);
                unsigned char *row = pool + slot * a.row_bytes;
                if (pos >= start && pos < end) {
                    quant_row<VEC, QM>(a, rowsp + (tb + (pos - start)) * a.out_row_bytes, row,
                                       slot);
                } else if (pos >= end && pos < zend) {
                    if (a.row_bytes % 16 == 0) {
                        for (uint32_t i = lane; i < a.row_bytes / 16; i += 64)
                            st_stream(u32x4(0), reinterpret_cast<u32x4 *>(row) + i);
                    } else {
                        for (uint32_t i = lane; i < a.row_bytes; i += 64)
                            st_stream((unsigned char)0, row + i);
                    }
                    if (lane == 0) {
                        a.qs_scales[slot] = 0.0f;
                        if (QM & 1)
                            a.qs_zero_points[slot] = 0;
                    }
                }
            }
        } else if constexpr (OP == Op::Scatter) {
            // Window w of absolute positions [w*rpc, (w+1)*rpc) of sequence s.
            const uint64_t w = udiv(start, a.div_rpc) + u;
            const uint64_t pos0 = w * rpc;
            const uint64_t q = udiv(w, a.div_upp);
            // slot of the window's first position in its page; byte offsets
            // inside a page are 64-bit (a page may exceed 4 GiB)
            const uint64_t slot0 = pos0 - q * P;
            const uint64_t phys = uni64(ld_idx<IdxT>(a.block_table, sp + q));
            const uint64_t end = start + len;
            unsigned char *page = pool + phys * P * a.row_bytes;
            const uint64_t wa = pos0 > start ? pos0 : start;
            const uint64_t wb = pos0 + rpc < end ? pos0 + rpc : end;
            if (wa < wb) {
                const unsigned char *from = rowsp + (tb + (wa - start)) * a.row_bytes;
                copy_span<U, VEC, NTL>(from, page + (slot0 + (wa - pos0)) * a.row_bytes,
                               (uint32_t)(wb - wa) * a.row_bytes);
            }
            if (a.zero_tail) {
                const uint64_t zend = udiv(end + P - 1, a.div_page) * P;
                const uint64_t za = pos0 > end ? pos0 : end;
                const uint64_t zb = pos0 + rpc < zend ? pos0 + rpc : zend;
                if (za < zb)
                    zero_span<VEC>(page + (slot0 + (za - pos0)) * a.row_bytes,
                                   (uint32_t)(zb - za) * a.row_bytes);
            }
        } else {
            const uint64_t t0 = (uint64_t)u * rpc;
            const uint32_t rows = (uint32_t)min64(rpc, len - t0);
            const uint32_t q = udiv32(u, a.div_upp);
            const uint32_t slot0 = (u - q * a.units_per_page) * rpc;
            const uint64_t phys = uni64(ld_idx<IdxT>(a.block_table, sp + q));
            const unsigned char *from = pool + (phys * P + slot0) * a.row_bytes;
            unsigned char *to = rowsp + (tb + t0) * a.out_row_bytes;
            if constexpr (OP == Op::Gather) {
                copy_span<U, VEC, NTL>(from, to, rows * a.row_bytes);
            } else if constexpr (QM >= 0) {
                const float *sl = QM == 0 ? a.scales[blockIdx.y] + phys * P + slot0 : nullptr;
                dequant_span_q<VEC, QM>(a, from, sl, phys * P + slot0, to, rows, tab);
            } else {
                dequant_span<VEC>(a, from, a.scales[blockIdx.y] + phys * P + slot0, to, rows);
            }
        }
    }
}

// ---- plan pass (more sequences than fit in LDS) ----------------------------------

template <typename IdxT, Op OP>
__global__ __launch_bounds__(kThreads) void plan_sum_kernel(Args a) {
    const uint32_t s0 = blockIdx.x * kPlanChunk;
    const uint32_t s1 = min32(s0 + kPlanChunk, a.num_seqs);
    const uint32_t per = kPlanChunk / kThreads;
    const uint32_t i0 = min32(s1, s0 + threadIdx.x * per);
    const uint32_t i1 = min32(s1, i0 + per);
    uint64_t u = 0, t = 0;
    for (uint32_t i = i0; i < i1; ++i) {
        const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
        const uint64_t st = (writes_pool(OP) && a.seq_start) ? ld_idx<IdxT>(a.seq_start, i) : 0;
        u += units_of<OP>(a, len, st);
        t += len;
    }
    uint64_t tu, tt;
    group_exclusive_scan(u, t, tu, tt);
    if (threadIdx.x == 0) {
        a.partials[2 * blockIdx.x] = tu;
        a.partials[2 * blockIdx.x + 1] = tt;
    }
}

// One workgroup: exclusive scan of the per-chunk totals, in place.
__global__ __launch_bounds__(kThreads) void plan_scan_kernel(uint64_t *partials, uint32_t chunks) {
    uint64_t cu = 0, ct = 0;
    for (uint32_t b = 0; b < chunks; b += kThreads) {
        const uint32_t i = b + threadIdx.x;
        uint64_t u = i < chunks ? partials[2 * i] : 0;
        uint64_t t = i < chunks ? partials[2 * i + 1] : 0;
        uint64_t tu, tt;
        group_exclusive_scan(u, t, tu, tt);
        if (i < chunks) {
            partials[2 * i] = cu + u;
            partials[2 * i + 1] = ct + t;
        }
        cu += tu;
        ct += tt;
    }
}

template <typename IdxT, Op OP>
__global__ __launch_bounds__(kThreads) void plan_write_kernel(Args a, uint32_t *unit_end,
                                                              uint64_t *tok_begin) {
    const uint32_t s0 = blockIdx.x * kPlanChunk;
    const uint32_t s1 = min32(s0 + kPlanChunk, a.num_seqs);
    scan_range<IdxT, OP>(a, s0, s1, a.partials[2 * blockIdx.x], a.partials[2 * blockIdx.x + 1],
                         unit_end, tok_begin);
}

// ---- validator -----------------------------------------------------------------------

struct VArgs {
    const void *block_table, *seq_ptr, *seq_lens, *seq_start;
    unsigned long long *ws;  // [0] min key, [1] token sum
    uint64_t num_pages, page_size, num_seqs, num_block_entries;
};

__global__ void validate_init_kernel(unsigned long long *ws) {
    if (threadIdx.x == 0) {
        ws[0] = ~0ull;
        ws[1] = 0ull;
    }
}

__device__ __forceinline__ unsigned long long vkey(uint64_t rank, uint64_t index) {
    return (rank << kKeyShift) | index;
}

// The checks that name item i (of max(K, S + 1) items), folded into the
// thread's smallest (check, index) key and its token sum.
template <typename IdxT>
__device__ __forceinline__ void validate_item(const VArgs &a, uint64_t i, unsigned long long &key,
                                              unsigned long long &sum) {
    const uint64_t S = a.num_seqs, K = a.num_block_entries;
    if (i == 0) {
        if (ld_idx<IdxT>(a.seq_ptr, 0) != 0)
            key = min64(key, vkey(kRankSeqPtrFirst, 0));
        if (ld_idx<IdxT>(a.seq_ptr, S) != K)
            key = min64(key, vkey(kRankSeqPtrLast, S));
    }
    if (i < S) {
        const uint64_t p0 = ld_idx<IdxT>(a.seq_ptr, i), p1 = ld_idx<IdxT>(a.seq_ptr, i + 1);
        if (p0 > p1)
            key = min64(key, vkey(kRankSeqPtrOrder, i));
        const uint64_t len = ld_idx<IdxT>(a.seq_lens, i);
        const uint64_t st = a.seq_start ? ld_idx<IdxT>(a.seq_start, i) : 0;
        if (p0 <= p1) {
            const uint64_t slice = p1 - p0;
            const uint64_t cap = __umul64hi(slice, a.page_size) ? ~0ull : slice * a.page_size;
            if (st > cap || len > cap - st)
                key = min64(key, vkey(kRankSeqLen, i));
        }
        sum += len;
    }
    if (i < K && ld_idx<IdxT>(a.block_table, i) >= a.num_pages)
        key = min64(key, vkey(kRankPageRange, i));
}

__device__ __forceinline__ void wave_fold(unsigned long long &key, unsigned long long &sum) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        key = min64(key, (unsigned long long)__shfl_xor(key, off, 64));
        sum += (unsigned long long)__shfl_xor(sum, off, 64);
    }
}

// One pass over max(K, S+1) items. Each item evaluates the checks that name
// its index; the smallest (check, index) key wins through atomicMin, which
// makes the report independent of scheduling.
template <typename IdxT>
__global__ __launch_bounds__(256) void validate_kernel(VArgs a) {
    const uint64_t S = a.num_seqs, K = a.num_block_entries;
    const uint64_t n = K > S + 1 ? K : S + 1;
    unsigned long long key = ~0ull, sum = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        validate_item<IdxT>(a, i, key, sum);
    wave_fold(key, sum);
    if ((threadIdx.x & 63) == 0) {
        if (key != ~0ull)
            atomicMin(&a.ws[0], key);
        if (sum)
            atomicAdd(&a.ws[1], sum);
    }
}

// Small descriptors: one workgroup evaluates every item and writes both result
// words itself, so no clearing kernel and no atomics are needed. `out` is
// the workspace or pinned host memory; system-scope stores make the words
// visible to the host once the kernel has finished.
constexpr uint32_t kValidateOneThreads = 1024;
template <typename IdxT>
__global__ __launch_bounds__(kValidateOneThreads) void validate_one_kernel(VArgs a,
                                                                           unsigned long long *out) {
    __shared__ unsigned long long wkey[kValidateOneThreads / 64], wsum[kValidateOneThreads / 64];
    const uint64_t S = a.num_seqs, K = a.num_block_entries;
    const uint64_t n = K > S + 1 ? K : S + 1;
    unsigned long long key = ~0ull, sum = 0;
    for (uint64_t i = threadIdx.x; i < n; i += kValidateOneThreads)
        validate_item<IdxT>(a, i, key, sum);
    wave_fold(key, sum);
    if ((threadIdx.x & 63) == 0) {
        wkey[threadIdx.x >> 6] = key;
        wsum[threadIdx.x >> 6] = sum;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (uint32_t w = 1; w < kValidateOneThreads / 64; ++w) {
            key = min64(key, wkey[w]);
            sum += wsum[w];
        }
        __hip_atomic_store(&out[0], key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&out[1], sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// ---- copy-on-write page copy ---------------------------------------------------------


struct PArgs {
    const void *src_pages, *dst_pages;
    uint64_t page_bytes;
    uint32_t page_size, chunks_per_page;
    unsigned char *pool[kMaxBatch];
    float *scales[kMaxBatch];
};

// Workgroup (x, m) copies chunk x % chunks_per_page of copy x / chunks_per_page
// in pool m (x in dispatch order by default; HP_PAGE_XCD gives each XCD a
// contiguous range of chunks instead); the chunk-0 workgroup also copies the
// page's slot scales. Every copy reads a page and writes another one exactly
// once: non-temporal both ways, U loads per lane in flight (exactly one chunk).
// Measured on MI355X, 1,024 copies of 128 KiB pages, cold caches / back to
// back: 4 KiB chunks in dispatch order 48.9 / 45.9 us, 4 KiB in XCD order
// 50.4 / 45.2, 8 KiB in XCD order 50.4 / 47.8, 16 KiB 55.0 / 50.9; through a
// contiguous table (pages 0..1023 to 1024..2047) 4 KiB in dispatch order
// 48.5 / 45.2 us, in XCD order 52.7 / 49.1.
template <typename IdxT, int VEC, int U>
__global__ __launch_bounds__(kThreads) void copy_pages_kernel(PArgs a) {
    const uint64_t x = group_order<HP_PAGE_XCD != 0>(blockIdx.x, gridDim.x);
    const uint64_t i = x / a.chunks_per_page;
    const uint32_t c = (uint32_t)(x - i * a.chunks_per_page);
    const uint64_t src = uni64(ld_idx<IdxT>(a.src_pages, i));
    const uint64_t dst = uni64(ld_idx<IdxT>(a.dst_pages, i));
    unsigned char *pool = a.pool[blockIdx.y];
    const uint64_t off = (uint64_t)c * kPageChunkBytes;
    const uint64_t left = a.page_bytes - off;
    const uint32_t n = (uint32_t)(left < kPageChunkBytes ? left : kPageChunkBytes);
    copy_span<U, VEC, true>(pool + src * a.page_bytes + off, pool + dst * a.page_bytes + off, n);
    float *scales = a.scales[blockIdx.y];
    if (scales && c == 0) {
        for (uint32_t t = threadIdx.x; t < a.page_size; t += kThreads)
            scales[dst * a.page_size + t] = scales[src * a.page_size + t];
    }
}

template <typename IdxT>
__global__ __launch_bounds__(256) void check_pages_kernel(const void *src_pages,
                                                          const void *dst_pages, uint64_t copies,
                                                          uint64_t num_pages,
                                                          unsigned long long *ws) {
    unsigned long long key = ~0ull;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < copies;
         i += (uint64_t)gridDim.x * blockDim.x) {
        if (ld_idx<IdxT>(src_pages, i) >= num_pages || ld_idx<IdxT>(dst_pages, i) >= num_pages)
            key = min64(key, vkey(kRankPageRange, i));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        key = min64(key, (unsigned long long)__shfl_xor(key, off, 64));
    if ((threadIdx.x & 63) == 0 && key != ~0ull)
        atomicMin(&ws[0], key);
}

// ---- host-side dispatch ----------------------------------------------------------------

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

template <typename IdxT, Op OP, int VEC, bool NTL, int QM = -1, int U = kCopyUnroll>
hipError_t launch_vec(const Args &a, bool fused, dim3 grid, uint32_t plan_chunks,
                      uint32_t *unit_end, uint64_t *tok_begin, hipStream_t stream) {
    const size_t qlds =
        (OP == Op::Dequant && (QM == 2 || QM == 3)) ? sizeof(QParam) * (size_t)a.quant_channels : 0;
    if (fused) {
        const size_t lds = lds_table_bytes(a.num_seqs) + qlds;
        hipLaunchKernelGGL((copy_kernel<IdxT, OP, VEC, true, NTL, QM, U>), grid,
                           dim3(block_threads(OP, U)), lds,
                           stream, a);
        return hipGetLastError();
    }
    if (plan_chunks) {  // 0: the plan arrays are already in the workspace
        hipLaunchKernelGGL((plan_sum_kernel<IdxT, OP>), dim3(plan_chunks), dim3(kThreads), 0, stream,
                           a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kThreads), 0, stream, a.partials,
                           plan_chunks);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        hipLaunchKernelGGL((plan_write_kernel<IdxT, OP>), dim3(plan_chunks), dim3(kThreads), 0,
                           stream, a, unit_end, tok_begin);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((copy_kernel<IdxT, OP, VEC, false, NTL, QM, U>), grid,
                       dim3(block_threads(OP, U)), qlds,
                       stream, a);
    return hipGetLastError();
}

template <typename IdxT, int VEC, int U>
hipError_t launch_quant(const Args &a, bool fused, dim3 grid, uint32_t chunks, uint32_t *ue,
                        uint64_t *tb, hipStream_t st, int qm) {
    constexpr Op OP = Op::ScatterQuant;
    switch (qm) {  // source type * 2 + asymmetric
    case 0: return launch_vec<IdxT, OP, VEC, false, 0, U>(a, fused, grid, chunks, ue, tb, st);
    case 1: return launch_vec<IdxT, OP, VEC, false, 1, U>(a, fused, grid, chunks, ue, tb, st);
    case 2: return launch_vec<IdxT, OP, VEC, false, 2, U>(a, fused, grid, chunks, ue, tb, st);
    case 3: return launch_vec<IdxT, OP, VEC, false, 3, U>(a, fused, grid, chunks, ue, tb, st);
    case 4: return launch_vec<IdxT, OP, VEC, false, 4, U>(a, fused, grid, chunks, ue, tb, st);
    default: return launch_vec<IdxT, OP, VEC, false, 5, U>(a, fused, grid, chunks, ue, tb, st);
    }
}

// Load policy per move (chosen on the host, measured on MI355X): a gather
// streams the pool only when the caller says no page is read twice; a scatter
// streams its source only when the move is larger than the Infinity Cache;
// dequant's 1:2 read:write mix reads through the cache.
template <typename IdxT, Op OP, int VEC>
hipError_t launch_policy(const Args &a, bool ntl, bool fused, dim3 grid, uint32_t chunks,
                         uint32_t *ue, uint64_t *tb, hipStream_t st, int qm, int u) {
    if constexpr (OP == Op::ScatterQuant) {
        if constexpr (VEC == 16) {
            if (u == 1)  // one wave per workgroup, one slot each
                return launch_quant<IdxT, VEC, 1>(a, fused, grid, chunks, ue, tb, st, qm);
        }
        // four waves per workgroup, a row each (U = 8)
        return launch_quant<IdxT, VEC, 8>(a, fused, grid, chunks, ue, tb, st, qm);
    } else if constexpr (OP == Op::Dequant) {
        switch (qm) {
        case 0: return launch_vec<IdxT, OP, VEC, false, 0>(a, fused, grid, chunks, ue, tb, st);
        case 1: return launch_vec<IdxT, OP, VEC, false, 1>(a, fused, grid, chunks, ue, tb, st);
        case 2: return launch_vec<IdxT, OP, VEC, false, 2>(a, fused, grid, chunks, ue, tb, st);
        case 3: return launch_vec<IdxT, OP, VEC, false, 3>(a, fused, grid, chunks, ue, tb, st);
        case 4: return launch_vec<IdxT, OP, VEC, false, 4>(a, fused, grid, chunks, ue, tb, st);
        case 5: return launch_vec<IdxT, OP, VEC, false, 5>(a, fused, grid, chunks, ue, tb, st);
        default: return launch_vec<IdxT, OP, VEC, false>(a, fused, grid, chunks, ue, tb, st);
        }
    } else if constexpr (VEC == 16) {
        // u: loads in flight per lane, the smallest of 2, 4, 8 covering a unit
        if (ntl) {
            if (u == 2)
                return launch_vec<IdxT, OP, VEC, true, -1, 2>(a, fused, grid, chunks, ue, tb, st);
            if (u == 4)
                return launch_vec<IdxT, OP, VEC, true, -1, 4>(a, fused, grid, chunks, ue, tb, st);
            return launch_vec<IdxT, OP, VEC, true, -1, 8>(a, fused, grid, chunks, ue, tb, st);
        }
        if (u == 2)
            return launch_vec<IdxT, OP, VEC, false, -1, 2>(a, fused, grid, chunks, ue, tb, st);
        if (u == 4)
            return launch_vec<IdxT, OP, VEC, false, -1, 4>(a, fused, grid, chunks, ue, tb, st);
        return launch_vec<IdxT, OP, VEC, false, -1, 8>(a, fused, grid, chunks, ue, tb, st);
    } else {
        if (ntl)
            return launch_vec<IdxT, OP, VEC, true>(a, fused, grid, chunks, ue, tb, st);
        return launch_vec<IdxT, OP, VEC, false>(a, fused, grid, chunks, ue, tb, st);
    }
}

template <typename IdxT, Op OP>
hipError_t launch_op(const Args &a, uint32_t vec, bool ntl, bool fused, dim3 grid,
                     uint32_t chunks, uint32_t *ue, uint64_t *tb, hipStream_t st, int qm, int u) {
    if constexpr (OP == Op::ScatterQuant) {
        if (vec == 16)  // 8 values per vector
            return launch_policy<IdxT, OP, 16>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        return launch_policy<IdxT, OP, 1>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
    } else if constexpr (OP == Op::Dequant) {
        switch (vec) {
        case 8: return launch_policy<IdxT, OP, 8>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        case 4: return launch_policy<IdxT, OP, 4>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        case 2: return launch_policy<IdxT, OP, 2>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        default: return launch_policy<IdxT, OP, 1>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        }
    } else {
        switch (vec) {
        case 16: return launch_policy<IdxT, OP, 16>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        case 8: return launch_policy<IdxT, OP, 8>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        case 4: return launch_policy<IdxT, OP, 4>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        case 2: return launch_policy<IdxT, OP, 2>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        default: return launch_policy<IdxT, OP, 1>(a, ntl, fused, grid, chunks, ue, tb, st, qm, u);
        }
    }
}

template <typename IdxT>
hipError_t launch_idx(const Args &a, Op op, uint32_t vec, bool ntl, bool fused, dim3 grid,
                      uint32_t chunks, uint32_t *ue, uint64_t *tb, hipStream_t st, int qm, int u) {
    switch (op) {
    case Op::Gather:
        return launch_op<IdxT, Op::Gather>(a, vec, ntl, fused, grid, chunks, ue, tb, st, -1, u);
    case Op::Scatter:
        return launch_op<IdxT, Op::Scatter>(a, vec, ntl, fused, grid, chunks, ue, tb, st, -1, u);
    case Op::ScatterQuant:
        return launch_op<IdxT, Op::ScatterQuant>(a, vec, ntl, fused, grid, chunks, ue, tb, st, qm, u);
    default:
        return launch_op<IdxT, Op::Dequant>(a, vec, ntl, fused, grid, chunks, ue, tb, st, qm, u);
    }
}

} // namespace

uint64_t plan_workspace_bytes(uint64_t num_seqs) {
    const uint64_t chunks = (num_seqs + kPlanChunk - 1) / kPlanChunk;
    return align256(8 * num_seqs) + align256(4 * num_seqs) + align256(16 * chunks);
}

hipError_t launch_copy(const CopyJob &job, hipStream_t stream) {
    // hipGetLastError reports the thread's last error from any HIP call; clear
    // what earlier calls (not ours) left so that the checks after each launch
    // see only that launch.
    (void)hipGetLastError();
    Args a = {};
    a.block_table = job.block_table;
    a.seq_ptr = job.seq_ptr;
    a.seq_lens = job.seq_lens;
    a.seq_start = job.seq_start;
    a.num_seqs = (uint32_t)job.num_seqs;
    a.page_size = job.page_size;
    a.rows_per_unit = job.rows_per_unit;
    a.units_per_page = job.page_size / job.rows_per_unit;
    a.units_per_group = job.units_per_group;
    a.row_bytes = (uint32_t)job.row_bytes;
    a.out_row_bytes = (uint32_t)job.out_row_bytes;
    a.zero_tail = job.zero_tail ? 1u : 0u;
    if (job.op == Op::Dequant)
        a.vecs_per_row = (uint32_t)(job.row_bytes / job.vec_bytes);
    a.div_vpr = make_div(a.vecs_per_row ? a.vecs_per_row : 1);
    a.quant_unsigned = job.quant_unsigned ? 1u : 0u;
    a.quant_channels = job.quant_channels;
    int qm = job.quant_ext ? (int)job.quant_mode : -1;
    if (qm >= 2 && job.quant_channels > kQuantLdsMax)
        qm += 2;  // table too large for LDS: read it from global memory
    if (job.op == Op::ScatterQuant)
        qm = (int)job.qs_src * 2 + (job.qs_asym ? 1 : 0);
    a.qs_scales = job.qs_scales;
    a.qs_zero_points = job.qs_zero_points;
    a.gate = job.gate;
    a.gate_tokens = job.gate_tokens;
    a.quant_scales = job.quant_scales;
    a.zero_points = job.zero_points;
    a.head_dim = job.head_dim ? job.head_dim : 1;
    a.div_hd = make_div(a.head_dim);
    a.div_rpc = make_div(job.rows_per_unit);
    a.div_page = make_div(job.page_size);
    a.div_upp = make_div(a.units_per_page);
    const bool fused = !job.plan;
    const uint64_t grid64 = (job.unit_bound + job.units_per_group - 1) / job.units_per_group;
    const uint32_t grid = (uint32_t)grid64;
    uint32_t chunks = 0;
    uint32_t *ue = nullptr;
    uint64_t *tb = nullptr;
    if (!fused) {
        unsigned char *ws = static_cast<unsigned char *>(job.workspace);
        const uint64_t S = job.num_seqs;
        chunks = (uint32_t)((S + kPlanChunk - 1) / kPlanChunk);
        tb = reinterpret_cast<uint64_t *>(ws);
        ue = reinterpret_cast<uint32_t *>(ws + align256(8 * S));
        a.partials = reinterpret_cast<uint64_t *>(ws + align256(8 * S) + align256(4 * S));
        a.g_unit_end = ue;
        a.g_tok_begin = tb;
    }
    // Loads in flight per lane for a gather or scatter with 16-byte vectors:
    // the smallest of 2, 4, 8 that covers one unit.
    const uint64_t per_lane = (job.rows_per_unit * job.row_bytes + (uint64_t)kThreads * 16 - 1) /
                              ((uint64_t)kThreads * 16);
    // Quantize-on-scatter: 1 for one wave per workgroup, else 8.
    const int u = job.op == Op::ScatterQuant ? (job.qs_wave_groups ? 1 : 8)
                  : per_lane <= 2                ? 2
                  : per_lane <= 4                ? 4
                                                 : 8;
    // The plan arrays depend only on the shared table: the plan kernels run
    // with the first launch only, later launches of a large batch reuse them.
    for (uint32_t first = 0; first < job.count; first += kMaxBatch, chunks = 0) {
        const uint32_t n = job.count - first < kMaxBatch ? job.count - first : kMaxBatch;
        for (uint32_t m = 0; m < n; ++m) {
            a.pool[m] = static_cast<unsigned char *>(job.pools[first + m]);
            a.rows[m] = static_cast<unsigned char *>(job.rows[first + m]);
            a.scales[m] = job.scales ? job.scales[first + m] : nullptr;
        }
        const dim3 g(grid, n);
        const hipError_t e =
            job.idx64 ? launch_idx<uint64_t>(a, job.op, job.vec_bytes, job.load_nt, fused, g, chunks,
                                             ue, tb, stream, qm, u)
                      : launch_idx<uint32_t>(a, job.op, job.vec_bytes, job.load_nt, fused, g, chunks,
                                             ue, tb, stream, qm, u);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename IdxT, int VEC>
hipError_t launch_pages(PArgs &a, const PageCopyJob &job, hipStream_t stream) {
    const uint64_t units = job.copies * a.chunks_per_page;
    for (uint32_t first = 0; first < job.count; first += kMaxBatch) {
        const uint32_t n = job.count - first < kMaxBatch ? job.count - first : kMaxBatch;
        for (uint32_t m = 0; m < n; ++m) {
            a.pool[m] = static_cast<unsigned char *>(job.pools[first + m]);
            a.scales[m] = job.scales ? job.scales[first + m] : nullptr;
        }
        // loads in flight per lane: the smallest of 1, 2, 4, 8 that covers a chunk
        constexpr int U = VEC < 16 ? kCopyUnroll
                          : kPageChunkBytes <= kThreads * 16     ? 1
                          : kPageChunkBytes <= 2 * kThreads * 16 ? 2
                          : kPageChunkBytes <= 4 * kThreads * 16 ? 4
                                                                 : 8;
        hipLaunchKernelGGL((copy_pages_kernel<IdxT, VEC, U>), dim3((uint32_t)units, n),
                           dim3(kThreads), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

template <typename IdxT>
hipError_t launch_pages_idx(PArgs &a, const PageCopyJob &job, hipStream_t st) {
    switch (job.vec_bytes) {
    case 16: return launch_pages<IdxT, 16>(a, job, st);
    case 8: return launch_pages<IdxT, 8>(a, job, st);
    case 4: return launch_pages<IdxT, 4>(a, job, st);
    case 2: return launch_pages<IdxT, 2>(a, job, st);
    default: return launch_pages<IdxT, 1>(a, job, st);
    }
}

hipError_t launch_copy_pages(const PageCopyJob &job, hipStream_t stream) {
    (void)hipGetLastError();  // see launch_copy
    PArgs a = {};
    a.src_pages = job.src_pages;
    a.dst_pages = job.dst_pages;
    a.page_bytes = job.page_bytes;
    a.page_size = job.page_size;
    a.chunks_per_page = (uint32_t)((job.page_bytes + kPageChunkBytes - 1) / kPageChunkBytes);
    return job.idx64 ? launch_pages_idx<uint64_t>(a, job, stream)
                     : launch_pages_idx<uint32_t>(a, job, stream);
}

hipError_t launch_check_pages(const PageCheckJob &job, hipStream_t stream) {
    (void)hipGetLastError();  // see launch_copy
    unsigned long long *ws = static_cast<unsigned long long *>(job.workspace);
    hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    uint64_t blocks = (job.copies + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (job.idx64)
        hipLaunchKernelGGL(check_pages_kernel<uint64_t>, dim3((uint32_t)blocks), dim3(256), 0,
                           stream, job.src_pages, job.dst_pages, job.copies, job.num_pages, ws);
    else
        hipLaunchKernelGGL(check_pages_kernel<uint32_t>, dim3((uint32_t)blocks), dim3(256), 0,
                           stream, job.src_pages, job.dst_pages, job.copies, job.num_pages, ws);
    return hipGetLastError();
}

// ---- write-disjointness of a scatter ----------------------------------------------
//
// [Hurray] Prefix Sharing lets slices name the same page, so a scatter's rows
// (or a row and a zeroed tail slot, [Hurray] Partial trailing page) can land
// in one slot, and the result would then depend on the order of the writes.
// On a descriptor that passed validation (every slot it names lies in the
// pool) one pass marks each written slot in a bitmap of num_pages *
// page_size bits and sets a second bitmap's bit for a slot it marks again;
// a second pass takes the smallest sequence that writes a slot of the second
// bitmap. A workgroup walks one sequence at a time.

struct DArgs {
    const void *block_table, *seq_ptr, *seq_lens, *seq_start;
    uint32_t *seen, *twice;          // num_pages * page_size bits each
    unsigned long long *answer;      // smallest clashing sequence, all ones if none
    uint64_t page_size, num_seqs, words;
    uint32_t zero_tail;
};

constexpr uint32_t kDisjointThreads = 256;

__global__ __launch_bounds__(kDisjointThreads) void disjoint_clear_kernel(DArgs a) {
    const uint64_t stride = (uint64_t)gridDim.x * kDisjointThreads;
    for (uint64_t i = (uint64_t)blockIdx.x * kDisjointThreads + threadIdx.x; i < a.words;
         i += stride) {
        a.seen[i] = 0;
        a.twice[i] = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *a.answer = ~0ull;
}

// f(slot) for every slot sequence s writes, spread over the workgroup's
// threads: its tokens' slots, then (zero_tail) the rest of the last token's page.
template <typename IdxT, typename F>
__device__ __forceinline__ void for_written_slots(const DArgs &a, uint64_t s, F &&f) {
    const uint64_t P = a.page_size;
    const uint64_t start = a.seq_start ? ld_idx<IdxT>(a.seq_start, s) : 0;
    const uint64_t L = ld_idx<IdxT>(a.seq_lens, s);
    const uint64_t base = ld_idx<IdxT>(a.seq_ptr, s);
    for (uint64_t i = threadIdx.x; i < L; i += kDisjointThreads) {
        const uint64_t t = start + i;
        f(ld_idx<IdxT>(a.block_table, base + t / P) * P + t % P);
    }
    if (a.zero_tail && L > 0) {
        const uint64_t last = start + L - 1;
        const uint64_t page = ld_idx<IdxT>(a.block_table, base + last / P);
        for (uint64_t r = last % P + 1 + threadIdx.x; r < P; r += kDisjointThreads)
            f(page * P + r);
    }
}

template <typename IdxT>
__global__ __launch_bounds__(kDisjointThreads) void disjoint_mark_kernel(DArgs a) {
    for (uint64_t s = blockIdx.x; s < a.num_seqs; s += gridDim.x)
        for_written_slots<IdxT>(a, s, [&](uint64_t slot) {
            const uint32_t bit = 1u << (slot & 31);
            if (atomicOr(&a.seen[slot >> 5], bit) & bit)
                atomicOr(&a.twice[slot >> 5], bit);
        });
}

template <typename IdxT>
__global__ __launch_bounds__(kDisjointThreads) void disjoint_find_kernel(DArgs a) {
    for (uint64_t s = blockIdx.x; s < a.num_seqs; s += gridDim.x) {
        bool hit = false;
        for_written_slots<IdxT>(a, s, [&](uint64_t slot) {
            hit |= ((a.twice[slot >> 5] >> (slot & 31)) & 1u) != 0;
        });
        if (hit)
            atomicMin(a.answer, (unsigned long long)s);
    }
}

hipError_t launch_disjoint(const DisjointJob &job, hipStream_t stream) {
    DArgs a;
    unsigned char *ws = static_cast<unsigned char *>(job.workspace);
    a.block_table = job.block_table;
    a.seq_ptr = job.seq_ptr;
    a.seq_lens = job.seq_lens;
    a.seq_start = job.seq_start;
    a.words = disjoint_words(job.num_pages, job.page_size);
    a.seen = reinterpret_cast<uint32_t *>(ws + kDisjointBitmaps);
    a.twice = a.seen + a.words;
    a.answer = reinterpret_cast<unsigned long long *>(ws + kDisjointAnswer);
    a.page_size = job.page_size;
    a.num_seqs = job.num_seqs;
    a.zero_tail = job.zero_tail;
    (void)hipGetLastError();  // see launch_copy
    uint64_t clear = (a.words + kDisjointThreads - 1) / kDisjointThreads;
    clear = clear < 1 ? 1 : clear > 4096 ? 4096 : clear;
    hipLaunchKernelGGL(disjoint_clear_kernel, dim3((uint32_t)clear), dim3(kDisjointThreads), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || job.num_seqs == 0)
        return e;
    const uint32_t groups = (uint32_t)(job.num_seqs < 65536 ? job.num_seqs : 65536);
    if (job.idx64)
        hipLaunchKernelGGL(disjoint_mark_kernel<uint64_t>, dim3(groups), dim3(kDisjointThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL(disjoint_mark_kernel<uint32_t>, dim3(groups), dim3(kDisjointThreads),
                           0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (job.idx64)
        hipLaunchKernelGGL(disjoint_find_kernel<uint64_t>, dim3(groups), dim3(kDisjointThreads),
                           0, stream, a);
    else
        hipLaunchKernelGGL(disjoint_find_kernel<uint32_t>, dim3(groups), dim3(kDisjointThreads),
                           0, stream, a);
    return hipGetLastError();
}

hipError_t launch_validate(const ValidateJob &job, hipStream_t stream) {
    VArgs a;
    a.block_table = job.block_table;
    a.seq_ptr = job.seq_ptr;
    a.seq_lens = job.seq_lens;
    a.seq_start = job.seq_start;
    a.ws = static_cast<unsigned long long *>(job.workspace);
    a.num_pages = job.num_pages;
    a.page_size = job.page_size;
    a.num_seqs = job.num_seqs;
    a.num_block_entries = job.num_block_entries;
    (void)hipGetLastError();  // see launch_copy
    const uint64_t n = job.num_block_entries > job.num_seqs + 1 ? job.num_block_entries
                                                                 : job.num_seqs + 1;
    if (n <= kValidateOneItems) {
        unsigned long long *out = static_cast<unsigned long long *>(job.result ? job.result
                                                                               : job.workspace);
        if (job.idx64)
            hipLaunchKernelGGL(validate_one_kernel<uint64_t>, dim3(1), dim3(kValidateOneThreads),
                               0, stream, a, out);
        else
            hipLaunchKernelGGL(validate_one_kernel<uint32_t>, dim3(1), dim3(kValidateOneThreads),
                               0, stream, a, out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(validate_init_kernel, dim3(1), dim3(64), 0, stream, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    if (job.idx64)
        hipLaunchKernelGGL(validate_kernel<uint64_t>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(validate_kernel<uint32_t>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace hp
